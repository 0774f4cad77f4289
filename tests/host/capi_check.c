/*
 * The C ABI used from plain C: device buffers from hipMalloc, pointer
 * arrays on the stack, the default stream, no torch.  Built into a shared
 * library that the GPU tests load and call in-process (capi_check()).
 *
 * Expected values are exact and computed here on the host: int32 sum
 * (two's-complement wrap) and max, where every schedule gives the same
 * result.  Also checked: in-place calls, the argument errors (misaligned,
 * overlapping, null, uninitialised), count 0, emu_tree_topology on the
 * intra-node chain, emu_buffer_layout placement, reduce-scatter and
 * all-gather, and emu_strerror.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "emu_comm.h"

#define MAXR 16

static char* g_msg;
static int g_len;

static int fail(const char* what, int code) {
  snprintf(g_msg, (size_t)g_len, "%s (code %d: %s)", what, code, emu_strerror(code));
  return 1;
}

static int32_t input_value(int r, size_t i) { return (int32_t)((uint32_t)(r + 1) * 2654435761u + (uint32_t)i * 40503u); }

static int run_case(int n, int m, int algo, int nch, size_t chunk, size_t count, int op, int inplace) {
  void* send[MAXR];
  void* recv[MAXR];
  int32_t* host = (int32_t*)malloc(count * sizeof(int32_t));
  int32_t* want = (int32_t*)malloc(count * sizeof(int32_t));
  int rc = 0;
  for (size_t i = 0; i < count; ++i) {
    uint32_t s = 0;
    int32_t mx = INT32_MIN;
    for (int r = 0; r < n; ++r) {
      const int32_t v = input_value(r, i);
      s += (uint32_t)v;
      if (v > mx) mx = v;
    }
    want[i] = op == EMU_SUM ? (int32_t)s : mx;
  }
  for (int r = 0; r < n; ++r) {
    if (hipMalloc(&send[r], count * sizeof(int32_t)) != hipSuccess) return fail("hipMalloc", EMU_ERR_HIP);
    recv[r] = send[r];
    if (!inplace && hipMalloc(&recv[r], count * sizeof(int32_t)) != hipSuccess) return fail("hipMalloc", EMU_ERR_HIP);
    for (size_t i = 0; i < count; ++i) host[i] = input_value(r, i);
    if (hipMemcpy(send[r], host, count * sizeof(int32_t), hipMemcpyHostToDevice) != hipSuccess)
      return fail("hipMemcpy", EMU_ERR_HIP);
  }
  int e = emu_comm_init(n, m, algo, nch, chunk);
  if (e) return fail("emu_comm_init", e);
  e = emu_allreduce((const void* const*)send, recv, count, EMU_INT32, op, NULL);
  if (e) return fail("emu_allreduce", e);
  if (hipDeviceSynchronize() != hipSuccess) return fail("hipDeviceSynchronize", EMU_ERR_HIP);
  for (int r = 0; r < n && !rc; ++r) {
    if (hipMemcpy(host, recv[r], count * sizeof(int32_t), hipMemcpyDeviceToHost) != hipSuccess)
      return fail("hipMemcpy", EMU_ERR_HIP);
    for (size_t i = 0; i < count; ++i)
      if (host[i] != want[i]) {
        snprintf(g_msg, (size_t)g_len, "n=%d m=%d algo=0x%x nch=%d count=%zu op=%d inplace=%d: rank %d element %zu is %d, want %d",
                 n, m, algo, nch, count, op, inplace, r, i, host[i], want[i]);
        rc = 1;
        break;
      }
  }
  for (int r = 0; r < n; ++r) {
    if (recv[r] != send[r]) (void)hipFree(recv[r]);
    (void)hipFree(send[r]);
  }
  free(host);
  free(want);
  return rc;
}

static int check_errors(void) {
  void* buf = NULL;
  const size_t count = 1024;
  if (hipMalloc(&buf, 8 * count * sizeof(int32_t) + 64) != hipSuccess) return fail("hipMalloc", EMU_ERR_HIP);
  char* b = (char*)buf;
  void* send[4];
  void* recv[4];
  for (int r = 0; r < 4; ++r) {
    send[r] = b + (size_t)r * count * sizeof(int32_t);
    recv[r] = b + (size_t)(4 + r) * count * sizeof(int32_t);
  }
  int e = emu_comm_init(4, 2, EMU_ALGO_TREE, 2, 4096);
  if (e) return fail("emu_comm_init", e);
  /* misaligned pointer */
  void* bad[4] = {send[0], send[1], send[2], b + 4};
  e = emu_allreduce((const void* const*)send, bad, count, EMU_INT32, EMU_SUM, NULL);
  if (e != EMU_ERR_INVALID_ARGUMENT) return fail("misaligned receive buffer accepted", e);
  /* rank 1 receives into rank 0's input */
  void* overlap[4] = {recv[0], send[0], recv[2], recv[3]};
  e = emu_allreduce((const void* const*)send, overlap, count, EMU_INT32, EMU_SUM, NULL);
  if (e != EMU_ERR_INVALID_ARGUMENT) return fail("overlapping buffers accepted", e);
  e = emu_allreduce(NULL, recv, count, EMU_INT32, EMU_SUM, NULL);
  if (e != EMU_ERR_INVALID_ARGUMENT) return fail("NULL send array accepted", e);
  e = emu_allreduce((const void* const*)send, recv, count, 99, EMU_SUM, NULL);
  if (e != EMU_ERR_INVALID_ARGUMENT) return fail("unknown dtype accepted", e);
  /* count 0: success and nothing written */
  if (hipMemset(recv[0], 0x5A, count * sizeof(int32_t)) != hipSuccess) return fail("hipMemset", EMU_ERR_HIP);
  e = emu_allreduce((const void* const*)send, recv, 0, EMU_INT32, EMU_SUM, NULL);
  if (e) return fail("count 0", e);
  if (hipDeviceSynchronize() != hipSuccess) return fail("hipDeviceSynchronize", EMU_ERR_HIP);
  uint32_t word = 0;
  if (hipMemcpy(&word, recv[0], sizeof(word), hipMemcpyDeviceToHost) != hipSuccess) return fail("hipMemcpy", EMU_ERR_HIP);
  if (word != 0x5A5A5A5Au) return fail("count 0 wrote the output", 0);
  /* chain of 2 ranks per node: rank 1 hangs below rank 0 */
  int up = 0, down[3] = {0, 0, 0};
  e = emu_tree_topology(0, 1, &up, down);
  if (e) return fail("emu_tree_topology", e);
  if (up != 0 || down[0] != -1 || down[1] != -1 || down[2] != -1) return fail("rank 1 record", 0);
  if (emu_tree_topology(2, 0, &up, down) != EMU_ERR_INVALID_ARGUMENT) return fail("channel 2 of 2 accepted", 0);
  e = emu_comm_destroy();
  if (e) return fail("emu_comm_destroy", e);
  e = emu_allreduce((const void* const*)send, recv, count, EMU_INT32, EMU_SUM, NULL);
  if (e != EMU_ERR_NOT_INITIALIZED) return fail("call after destroy", e);
  if (!emu_strerror(EMU_ERR_HIP) || !emu_strerror(12345)) return fail("emu_strerror", 0);
  (void)hipFree(buf);
  return 0;
}

/* Rank buffers placed by emu_buffer_layout in one pool; then reduce-scatter
 * and all-gather on the same communicator. */
static int check_layout_and_halves(void) {
  const int n = 8;
  const size_t block = 4096 + 4;      /* elements per block: 16-byte multiple */
  const size_t total = block * (size_t)n;
  size_t off[2 * 8], pool_bytes = 0;
  int e = emu_buffer_layout(2 * (size_t)n, total * sizeof(int32_t), off, &pool_bytes);
  if (e) return fail("emu_buffer_layout", e);
  void* pool = NULL;
  if (hipMalloc(&pool, pool_bytes) != hipSuccess) return fail("hipMalloc", EMU_ERR_HIP);
  void* send[8];
  void* mid[8];
  void* out[8];
  int32_t* host = (int32_t*)malloc(total * sizeof(int32_t));
  for (int r = 0; r < n; ++r) {
    send[r] = (char*)pool + off[r];
    out[r] = (char*)pool + off[n + r];
    mid[r] = (char*)out[r] + (size_t)r * block * sizeof(int32_t);   /* in-place all-gather source */
    for (size_t i = 0; i < total; ++i) host[i] = input_value(r, i);
    if (hipMemcpy(send[r], host, total * sizeof(int32_t), hipMemcpyHostToDevice) != hipSuccess)
      return fail("hipMemcpy", EMU_ERR_HIP);
  }
  e = emu_comm_init(n, 1, EMU_ALGO_RING, 4, 8192);
  if (e) return fail("emu_comm_init", e);
  e = emu_reduce_scatter((const void* const*)send, mid, block, EMU_INT32, EMU_SUM, NULL);
  if (e) return fail("emu_reduce_scatter", e);
  e = emu_all_gather((const void* const*)mid, out, block, EMU_INT32, NULL);
  if (e) return fail("emu_all_gather", e);
  if (hipDeviceSynchronize() != hipSuccess) return fail("hipDeviceSynchronize", EMU_ERR_HIP);
  int rc = 0;
  for (int r = 0; r < n && !rc; ++r) {
    if (hipMemcpy(host, out[r], total * sizeof(int32_t), hipMemcpyDeviceToHost) != hipSuccess)
      return fail("hipMemcpy", EMU_ERR_HIP);
    for (size_t i = 0; i < total; ++i) {
      uint32_t s = 0;
      for (int k = 0; k < n; ++k) s += (uint32_t)input_value(k, i);
      if (host[i] != (int32_t)s) {
        snprintf(g_msg, (size_t)g_len, "reduce-scatter + all-gather: rank %d element %zu is %d, want %d", r, i,
                 host[i], (int32_t)s);
        rc = 1;
        break;
      }
    }
  }
  free(host);
  (void)hipFree(pool);
  return rc;
}

int capi_check(char* msg, int len) {
  g_msg = msg;
  g_len = len;
  msg[0] = '\0';
  static const int modes[] = {EMU_MODE_STEPWISE, EMU_MODE_FUSED, EMU_PROTO_LL, EMU_TRANSPORT_DEVICE};
  for (int k = 0; k < 4; ++k)
    for (int t = 0; t < 2; ++t) {
      const int algo = (t == 0 ? EMU_ALGO_RING : EMU_ALGO_TREE) | modes[k];
      if (t == 1 && modes[k] == EMU_TRANSPORT_DEVICE) continue;   /* ring only */
      if (run_case(8, 1, algo, 4, 4096, 10007, EMU_SUM, 0)) return 1;
      if (run_case(6, 3, algo, 3, 1024, 5003, EMU_MAX, 1)) return 1;
      if (run_case(16, 16, algo, 2, 512, 3001, EMU_SUM, 1)) return 1;
    }
  if (check_errors()) return 1;
  if (check_layout_and_halves()) return 1;
  emu_comm_destroy();
  snprintf(msg, (size_t)len, "ok");
  return 0;
}
