"""emucomm: an MI355X-native emulator of the NCCL-style all-reduce data path.

N virtual ranks keep their buffers in one GPU's HBM.  The work sits in the
C-ABI library ``libemucomm.so`` (declared in ``include/emu_comm.h``); this
package only marshals arguments to it (``emucomm``) and draws seeded
synthetic inputs (``inputs``).  Importing the package loads nothing; the
library is loaded on first use and a missing library is an error.
"""

__all__ = ["emucomm", "inputs"]
