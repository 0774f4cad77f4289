/*
 * emu_comm.h - C ABI of libemucomm: an all-reduce data-path emulator for
 * N virtual ranks whose buffers all live in one GPU's HBM (AMD MI355X,
 * gfx950).
 *
 * The operation is the all-reduce of the NCCL public call as described on
 * the page "NCCL 内部机制：一次 AllReduce 如何变成拓扑图、Channel 与 GPU
 * Kernel" (section on the public API: send buffer, receive buffer, element
 * count, data type, reduction operator, communicator, stream; the call only
 * enqueues work on the stream).  Here every virtual rank has its own send and
 * receive buffer and one call reduces all of them.  The schedules are those
 * of "NCCL 专家课程 13：Tree、双树、层次化连接与真实交叉区间" (tree
 * reduce-up / broadcast-down, sections "先固定方向" and "runTreeSplit 如何流水";
 * double binary tree, section "双树：偶数 mirror，奇数 shift"; intra-node chain,
 * section "节点内先形成链") and of "all-reduce 每张卡要发多少数据? ring 和 tree
 * 有什么区别?" (ring reduce-scatter + all-gather, Figure 1 and section "手撕
 * 代码").
 *
 * One process-global communicator (the calls take no handle).  Not
 * thread-safe: the caller serialises calls.  Every function returns an
 * emu_result code; nothing throws or aborts across this boundary.
 */
#ifndef EMU_COMM_H
#define EMU_COMM_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Algorithms (low byte of `algo`).  TREE on one node is the intra-node
 * chain; on several nodes it is the chain inside each node plus the double
 * binary tree across node heads (by default local rank 0 of every node; see
 * emu_comm_init_graph for other chain orders and head patterns). */
#define EMU_ALGO_RING 0
#define EMU_ALGO_TREE 1
/* AUTO: each all-reduce runs the ring or the tree, whichever the cost model
 * (emu_predict_us) predicts faster for its size; reduce-scatter and
 * all-gather always run on the ring. */
#define EMU_ALGO_AUTO 2
/* Execution mode, OR-ed into `algo`.
 * STEPWISE (default): every ring step / tree hop runs as a receive-reduce-
 *   copy between virtual ranks through step FIFO slots, as the pages'
 *   primitives do.
 * FUSED: one pass that reads every rank's input once, evaluates each
 *   element in the schedule's exact order, and writes every rank's output.
 * Both give bit-identical results. */
#define EMU_MODE_STEPWISE 0x000
#define EMU_MODE_FUSED 0x100
/* Protocol of the stepwise all-reduce, OR-ed into `algo` (page "NCCL 内部
 * 机制：一次 AllReduce 如何变成拓扑图、Channel 与 GPU Kernel", sections
 * "Simple：有效载荷效率与大消息吞吐" and "LL：用更高的元数据比例换低延迟").
 * SIMPLE (default): a step's data goes through a FIFO slot and the ranks
 *   meet at a barrier after every step.
 * LL: every 8-byte FIFO word carries 4 data bytes and 4 flag bytes (the
 *   item's sequence number), written and read as one access; a rank polls
 *   the words it reads until they carry the flag it expects and publishes
 *   how many items it consumed, so the writer knows when a slot is free.
 *   No barriers between steps.  Stepwise mode only, at most 16 ranks (one
 *   64-lane wave per rank); reduce-scatter and all-gather on such a
 *   communicator run SIMPLE.  Same results, bit for bit.  Every wait is
 *   bounded: a call whose wait expires is abandoned, its outputs are
 *   undefined, and emu_protocol_status reports it. */
#define EMU_PROTO_SIMPLE 0x000
#define EMU_PROTO_LL 0x200
/* Transport of the stepwise ring all-reduce, OR-ed into `algo` (page "NCCL
 * 内部机制：…", sections "Chunk、slice、step 是三个尺度" and "Ring：带宽友
 * 好…": one CTA per channel on every GPU, steps handed over through FIFO
 * buffers).  DEVICE: every (channel, ring position) is a workgroup of its
 * own, all resident at once (a cooperative launch), and a step's data
 * travels through FIFOs in device memory, slice by slice, made
 * visible across the chip's L2 caches: with EMU_PROTO_SIMPLE by a release
 * fence plus a tail counter, with EMU_PROTO_LL by flag-in-line 8-byte words
 * (any nranks).  Ring only (EMU_ALGO_RING, stepwise); reduce-scatter and
 * all-gather on such a communicator run the one-workgroup stepwise kernels.
 * Same results, bit for bit.  The FIFOs and counters (per communicator and
 * device, nchannels * nranks FIFOs of twice the slices a chunk spans; a
 * slice is 32 KiB with SIMPLE, 8 KiB of data in 16 KiB of flagged words with
 * LL; at most 4 GiB) are created on the first
 * all-reduce and reused: calls of one communicator must not overlap (order
 * them on one stream).  The first call fails with EMU_ERR_INVALID_ARGUMENT
 * when nchannels * nranks workgroups cannot be resident at once or the
 * FIFOs would exceed 4 GiB.  Every wait is bounded; an abandoned call
 * leaves its outputs undefined, later calls do nothing until
 * emu_protocol_status has reported it (and cleared the FIFOs). */
#define EMU_TRANSPORT_DEVICE 0x400

/* Element types. */
#define EMU_INT32 0
#define EMU_INT64 1
#define EMU_FLOAT32 2
#define EMU_FLOAT16 3
#define EMU_BFLOAT16 4

/* Reduction operators.  Sum: integers wrap; floats are rounded to the
 * buffer type after every hop (f16/bf16: exact f32 add, then round to
 * nearest even), subnormals kept, overflow gives infinity.  Max: float max
 * orders -0 below +0, so its result does not depend on the order.  Float
 * inputs must not hold NaN (a NaN result, or a NaN input to max, is outside
 * the contract: its bits are unspecified). */
#define EMU_SUM 0
#define EMU_MAX 1

/* Result codes. */
#define EMU_SUCCESS 0
#define EMU_ERR_INVALID_ARGUMENT 1
#define EMU_ERR_NOT_INITIALIZED 2
#define EMU_ERR_INTERNAL 3
#define EMU_ERR_HIP 4

/* Intra-node head patterns (page "NCCL 专家课程 13", section "节点内先形成
 * 链"; page "NCCL代码分析", section "Tree搜索"): which chain positions of a
 * node carry its node-level edges.  The edge to the parent node always
 * leaves from chain position 0; the edges from the child nodes arrive at
 *   TREE           position 0 (child0 and child1),
 *   SPLIT_TREE     position 1 (child0 and child1),
 *   BALANCED_TREE  position 1 (child0) and position 0 (child1).
 * SPLIT_TREE and BALANCED_TREE need at least two ranks per node. */
#define EMU_PATTERN_TREE 0
#define EMU_PATTERN_SPLIT_TREE 1
#define EMU_PATTERN_BALANCED_TREE 2

/* Limits. */
#define EMU_MAX_RANKS 64
#define EMU_MAX_CHANNELS 64

/* Environment.  The library reads no environment variable unless EMU_DEBUG
 * is set.  With EMU_DEBUG set, tuning knobs (EMU_FUSED_BLOCKS_PER_CU,
 * EMU_FUSED_XCD_RUNS, EMU_TREE_TASKS_PER_CU, EMU_TREE_PIECE_MIN,
 * EMU_TREE_LONG_PIECES, EMU_STEP_GROUP, EMU_XWG_SLOTS)
 * and test hooks that shorten the bounded waits (EMU_LL_SPIN_LIMIT,
 * EMU_XWG_SPIN_LIMIT) override the built-in values of plans built after
 * they are set; EMU_DEBUG=1 also prints every tree record at init.  They
 * are for debugging and measurement only. */

/*
 * emu_comm_init - build the communicator: per-channel tree records for
 * `nranks` virtual ranks on `nnodes` nodes (ranks are node-major:
 * rank = node * (nranks/nnodes) + local), the channel count and the chunk
 * size.
 *   nranks      1..EMU_MAX_RANKS
 *   nnodes      >= 1, divides nranks
 *   algo        EMU_ALGO_RING, EMU_ALGO_TREE or EMU_ALGO_AUTO, optionally
 *               | EMU_MODE_FUSED or | EMU_PROTO_LL (not both; LL needs
 *               nranks <= 16), or EMU_ALGO_RING | EMU_TRANSPORT_DEVICE,
 *               optionally | EMU_PROTO_LL (any nranks)
 *   nchannels   1..EMU_MAX_CHANNELS.  The message is split into nchannels
 *               disjoint ranges (page "NCCL 专家课程 13", section "前置知识");
 *               the first ceil(nchannels/2) channels use tree 0, the others
 *               tree 1 (the duplicated channel records of section "节点内先
 *               形成链").
 *   chunk_bytes > 0, a multiple of 16, at most 1 GiB.  Tree: chunk size
 *               inside a channel; ring: each loop covers nranks chunks.
 * Host only: touches no GPU (device resources are created on the first
 * emu_allreduce), except that when more than 16 configurations have been
 * initialised in the process the cached ones are dropped, which waits for
 * the device to go idle before freeing their tables.  Replaces any previous
 * communicator; re-initialising with arguments used before reuses the
 * tables built for them.
 * Errors: EMU_ERR_INVALID_ARGUMENT for out-of-range arguments (state left
 * unchanged); EMU_ERR_INTERNAL if a tree record overflows (cannot happen
 * within the limits above).
 */
int emu_comm_init(int nranks, int nnodes, int algo, int nchannels, size_t chunk_bytes);

/*
 * emu_comm_init_graph - emu_comm_init with per-channel rank orders and a head
 * pattern, the two things a graph search hands to the tree and ring builders
 * (page "NCCL 专家课程 13", section "节点内先形成链", and the per-channel
 * chain table of section "从 GRAPH 日志复原 active tree").
 *   pattern  EMU_PATTERN_TREE, EMU_PATTERN_SPLIT_TREE or
 *            EMU_PATTERN_BALANCED_TREE
 *   intra    NULL (every channel in identity order), or nchannels * nranks
 *            ints: row c lists node 0's ranks in channel c's chain order,
 *            then node 1's, and so on; each node's part is a permutation of
 *            that node's ranks.  Tree: the chain inside each node follows
 *            the order (parent = previous, first child = next).  Ring: the
 *            ring of channel c visits the ranks in the row's order, node
 *            after node.  Read during the call only.
 * The other arguments, the caching and the errors are those of
 * emu_comm_init; EMU_ERR_INVALID_ARGUMENT also for an unknown pattern, a
 * pattern that needs two ranks per node on one-rank nodes, or a row that is
 * not a node-by-node permutation.  emu_comm_init(...) is
 * emu_comm_init_graph(..., EMU_PATTERN_TREE, NULL).
 */
int emu_comm_init_graph(int nranks, int nnodes, int algo, int nchannels, size_t chunk_bytes,
                        int pattern, const int* intra);

/*
 * emu_allreduce - enqueue one all-reduce on `stream` (a hipStream_t; NULL is
 * the default stream) and return.  Completion is observed by synchronising
 * the stream.
 *   sendbufs  host array of nranks device pointers; sendbufs[r] holds
 *             `count` elements of virtual rank r
 *   recvbufs  host array of nranks device pointers, the outputs; after
 *             completion every recvbufs[r][0..count) holds the same bits.
 *             recvbufs[r] == sendbufs[r] (in place) is allowed; any other
 *             overlap between buffers is invalid.
 *   count     elements per rank; 0 is a successful no-op
 *   dtype     EMU_INT32 .. EMU_BFLOAT16;  op  EMU_SUM or EMU_MAX
 * Every pointer must be non-NULL and 16-byte aligned.  The host arrays are
 * read during the call only; the device buffers must stay alive until the
 * stream work completes.  The caller owns all buffers and the stream; the
 * library owns its tables and device workspace.
 * count * element size must not exceed 2^40 bytes.
 * Errors (checked before anything is enqueued): EMU_ERR_NOT_INITIALIZED,
 * EMU_ERR_INVALID_ARGUMENT; EMU_ERR_HIP when the runtime refuses an
 * allocation, copy or launch.  Faults inside kernels surface at the stream
 * synchronisation.
 * Graph capture: the first call for a (count, dtype, op) on a device builds
 * that shape's tables (device allocation and a synchronous copy), so it must
 * run outside stream capture; every later call is exactly one kernel launch
 * on `stream` (no allocation, copy or memset) and may be captured in a HIP
 * graph and replayed.  The same holds for emu_reduce_scatter and
 * emu_all_gather.
 */
int emu_allreduce(const void* const sendbufs[], void* const recvbufs[], size_t count,
                  int dtype, int op, void* stream);

/*
 * emu_allreduce_noalloc - emu_allreduce for callers that cannot allocate
 * device memory: code under HIP stream capture, tight serving loops, and
 * harnesses that forbid hipMalloc.  Same arguments, results (bit for bit)
 * and errors as emu_allreduce.  It never calls hipMalloc, hipFree or any
 * allocating library routine: instead of tables in device buffers the
 * library allocates, it keeps the call's tables (and the LL status word) in
 * a static device array of EMU_NOALLOC_SCRATCH_BYTES bytes that every GPU
 * the library runs on holds from module load until the process ends.  Its
 * device address is looked up once per device, on the first call there.
 * A call copies its tables into the array with hipMemcpyAsync on `stream`
 * (skipped when the array already holds the same plan's tables), so the
 * caller passes only inputs and outputs.  Host memory for a new shape's
 * tables is taken on its first call and kept with the communicator.
 * Every call on a GPU shares that GPU's array, which keeps the last call's
 * tables: calls on one GPU that overlap in time (on different streams, or
 * from several threads) race; order them, e.g. on one stream.  Modes: fused
 * and stepwise (SIMPLE or LL; an LL abandon is reported by
 * emu_protocol_status).  Additional errors: EMU_ERR_INVALID_ARGUMENT for an
 * EMU_TRANSPORT_DEVICE communicator (its FIFOs are far larger than the
 * array) and for a call whose tables exceed the array (from about 512 MiB
 * per rank in fused mode; the stepwise tables are much smaller).
 */
#define EMU_NOALLOC_SCRATCH_BYTES (4u << 20)
int emu_allreduce_noalloc(const void* const sendbufs[], void* const recvbufs[], size_t count,
                          int dtype, int op, void* stream);

/*
 * emu_reduce_scatter - enqueue one reduce-scatter on `stream`: the first
 * half of the ring all-reduce run on its own (page "all-reduce 每张卡要发多少
 * 数据? ring 和 tree 有什么区别?", section "先弄清楚:每个概念是什么" and
 * Figure 1; page "NCCL代码分析", section "通讯时如何选择Channel": a ring-only
 * collective).  Uses the active communicator's channels, chunk size, rank
 * orders and mode; it runs on the ring whatever the communicator's `algo`.
 *   sendbufs[r]  nranks blocks of `recvcount` elements
 *   recvbufs[r]  `recvcount` elements: the reduction of block r over all
 *                ranks, folded in each channel's ring order starting at the
 *                position after rank r's and ending at rank r (the ring's
 *                reduce-scatter steps, arranged so that every rank finishes
 *                its own block), each op rounded as for emu_allreduce.
 *   recvcount    elements per block; recvcount * element size must be a
 *                multiple of 16 (every block 16-byte aligned); 0 is a no-op.
 *   dtype, op    as for emu_allreduce.
 * In place: recvbufs[r] == sendbufs[r] + r * recvcount elements.  Any other
 * overlap is invalid.  Pointers non-NULL and 16-byte aligned; nranks *
 * recvcount * element size at most 2^40 bytes.  Ownership, asynchrony and
 * errors as for emu_allreduce.
 */
int emu_reduce_scatter(const void* const sendbufs[], void* const recvbufs[], size_t recvcount,
                       int dtype, int op, void* stream);

/*
 * emu_all_gather - enqueue one all-gather on `stream`: the second half of
 * the ring all-reduce run on its own (same passages; ring only).  Every
 * rank's output gets rank k's `sendcount` input elements in block k, bit
 * for bit.
 *   sendbufs[r]  `sendcount` elements
 *   recvbufs[r]  nranks blocks of `sendcount` elements
 *   sendcount    sendcount * element size must be a multiple of 16; 0 is a
 *                no-op.
 * In place: sendbufs[r] == recvbufs[r] + r * sendcount elements.  Other
 * rules as for emu_reduce_scatter.
 */
int emu_all_gather(const void* const sendbufs[], void* const recvbufs[], size_t sendcount, int dtype,
                   void* stream);

/*
 * Algorithm selection by a cost model: the pages' alpha-beta formulas (page
 * "NCCL 专家课程 13", section "理想成本模型"; page "all-reduce 每张卡要发多少
 * 数据?", section "α–β 模型") with per-(mode, algorithm) parameters.  For
 * S = count * element size bytes per rank on the active communicator (N
 * ranks, D the deepest channel tree):
 *   ring: 2(N-1) * alpha + 2(N-1)/N * S / bw
 *   tree: 2 * D * alpha  + 2 * S / bw
 * (microseconds; the fixed cost of a call is folded into alpha).  alpha
 * and bw are kept per (mode, algorithm) and per rank-count class: N <= 11,
 * 12 <= N <= 22, N >= 23 (centred on 8, 16 and 32 ranks; on one GPU the
 * cost per stage and per byte changes with the number of virtual ranks).
 * The defaults are least-squares fits to message-size sweeps measured on
 * MI355X at 8, 16 and 32 ranks.  Selection takes the smaller predicted
 * time, the ring on an exact tie (page "NCCL代码分析", section "通讯时如何选择
 * Channel": the algorithm of least predicted time is used).
 *
 * emu_set_cost_model - replace alpha (us per stage, >= 0) and bw (bytes per
 *   us, > 0) of `algo` (EMU_ALGO_RING or EMU_ALGO_TREE, optionally |
 *   EMU_MODE_FUSED) in every rank-count class; process-wide, host only.
 *   EMU_ERR_INVALID_ARGUMENT for other algorithms or values out of range
 *   (state unchanged).
 * emu_set_cost_model_ranks - the same for the class of `nranks` only (1 ..
 *   EMU_MAX_RANKS; 0 means every class).
 * emu_get_cost_model - alpha and bw of `algo` in the class of `nranks`.
 * emu_predict_us - the predicted time of one all-reduce of `count` elements of
 *   `dtype` with `algo` (as above) on the active communicator, into *us.
 * emu_select_algo - the algorithm an all-reduce of `count` elements of
 *   `dtype` runs on the active communicator, into *algo (EMU_ALGO_RING or
 *   EMU_ALGO_TREE; the fixed algorithm unless it was initialised with
 *   EMU_ALGO_AUTO, whose choice uses the communicator's mode).
 * Errors: EMU_ERR_NOT_INITIALIZED; EMU_ERR_INVALID_ARGUMENT for a NULL
 * output, unknown dtype or algorithm.
 */
int emu_set_cost_model(int algo, double alpha_us, double bw_bytes_per_us);
int emu_set_cost_model_ranks(int algo, int nranks, double alpha_us, double bw_bytes_per_us);
int emu_get_cost_model(int algo, int nranks, double* alpha_us, double* bw_bytes_per_us);
int emu_predict_us(int algo, size_t count, int dtype, double* us);
int emu_select_algo(size_t count, int dtype, int* algo);

/*
 * emu_tree_topology - the tree record of `rank` in `channel`: its parent
 * (*up, -1 at the root) and its three child slots (down[0..2], -1 when
 * empty), in the order they were filled (intra-node child first, then the
 * node-level child0, then child1).  Mirrors the tree record of page "NCCL
 * 专家课程 13", section "数据结构不是纯二叉树".  Valid after emu_comm_init
 * for either algorithm.  Host only.
 * Errors: EMU_ERR_NOT_INITIALIZED; EMU_ERR_INVALID_ARGUMENT for a channel or
 * rank out of range or a NULL pointer.
 */
int emu_tree_topology(int channel, int rank, int* up, int down[3]);

/*
 * emu_tree_depth - the depth field of the tree records: the pages'
 * approximation nranks/nnodes - 1 + floor(log2(nnodes)) (section "节点间
 * 连接"), metadata only.  Errors: EMU_ERR_NOT_INITIALIZED, NULL pointer.
 */
int emu_tree_depth(int* depth);

/*
 * emu_comm_destroy - free the communicator and every device resource the
 * library allocated (tables, FIFO workspaces, protocol status words).  Call
 * with no work of the library pending on any stream.  Destroying when
 * nothing is initialised succeeds.  Nothing is freed at process exit: what
 * a process still holds when it ends is reclaimed with the process (freeing
 * from exit-time destructors would race the HIP runtime's own teardown).
 */
int emu_comm_destroy(void);

/*
 * emu_device_memory - how many device allocations the library holds now,
 * and their total size in bytes (tables, FIFO workspaces, status words; not
 * the caller's buffers).  Zero after emu_comm_destroy.  Host only.
 * Errors: EMU_ERR_INVALID_ARGUMENT for a NULL pointer.
 */
int emu_device_memory(size_t* allocations, size_t* bytes);

/*
 * emu_protocol_status - whether an LL or EMU_TRANSPORT_DEVICE all-reduce on
 * the current device was abandoned (a wait expired) since the last query:
 * *abandoned = 1 or 0.  Waits for the device to go idle, then reads and
 * clears the flag (and, if it was set, every EMU_TRANSPORT_DEVICE FIFO
 * workspace on the device); host only, not for use under stream capture.  A correct schedule never
 * abandons: every wait is for data or space that an earlier step of another
 * rank provides.
 * Errors: EMU_ERR_INVALID_ARGUMENT for NULL; EMU_ERR_HIP if the runtime
 * fails.
 */
int emu_protocol_status(int* abandoned);

/*
 * emu_buffer_layout - where to place `nbufs` buffers of `bytes` bytes each
 * inside one device allocation so that HBM serves them evenly: buffer i
 * starts at offsets[i] = i * slot, with slot = bytes rounded up to 64 KiB,
 * plus 6 KiB.  Buffers that a collective reads or writes at the same offset
 * (the same element of every rank) then start at different positions
 * modulo 64 KiB instead of the same one.  The allocation needs *pool_bytes
 * bytes and a base aligned to 64 KiB.  The stagger was chosen on MI355X
 * for the best worst case over the all-reduce workloads (8 ranks at 16 to
 * 256 MiB, 15 and 16 ranks bf16, 4 x 8 ranks f16, i64 and f32; ring and
 * tree, fused and stepwise; two alternating rounds against staggers of 4,
 * 5 and 7 KiB): no leg below 66.7% of 8 TB/s fused or 62% stepwise, where
 * 4 KiB let the fused ring at 128 MiB per rank fall to 59% and the 16-rank
 * stepwise ring to 58%; it costs the 8-rank 64 MiB fused pass about 1%.
 * Host arithmetic only; the library works with buffers placed anywhere.
 * Errors: EMU_ERR_INVALID_ARGUMENT for nbufs == 0, NULL pointers, or a
 * pool size that does not fit in size_t.
 */
int emu_buffer_layout(size_t nbufs, size_t bytes, size_t offsets[], size_t* pool_bytes);

/*
 * emu_stream_probe - enqueue one pass of a 128-bit streaming kernel on
 * `stream`, for measurement: the same-run HBM rates that the collectives'
 * bandwidth is compared with (a copy of the same byte count is the pages'
 * usual yardstick; an all-reduce moves half reads and half writes, so its
 * practical ceiling lies between the read-only and write-only rates).
 * Whole 16-byte vectors, non-temporal, as the collectives access memory.
 *   kind   EMU_STREAM_READ: read `bytes` at src (dst: 16 bytes the kernel
 *          may write, practically never);  EMU_STREAM_WRITE: write `bytes`
 *          of a fixed pattern at dst (src unused);  EMU_STREAM_COPY: copy
 *          `bytes` from src to dst (no overlap)
 *   bytes  a multiple of 16; 0 is a no-op.  Pointers 16-byte aligned.
 * Errors: EMU_ERR_INVALID_ARGUMENT (unknown kind, NULL or misaligned
 * pointer, bytes not a multiple of 16, overlapping copy); EMU_ERR_HIP for
 * a launch failure.  Needs no communicator.
 */
#define EMU_STREAM_READ 0
#define EMU_STREAM_WRITE 1
#define EMU_STREAM_COPY 2
int emu_stream_probe(int kind, const void* src, void* dst, size_t bytes, void* stream);

/* emu_strerror - static description of a result code (never NULL). */
const char* emu_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* EMU_COMM_H */
