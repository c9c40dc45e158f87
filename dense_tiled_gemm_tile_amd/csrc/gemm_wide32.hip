// Wide streaming GEMM instances for fp32 operands (fp32 MFMA, full fp32
// products).  The 64-cycle fp32 MFMAs hide the copy and barrier overheads:
// 96 % of the fp32 MFMA peak at 4096^3.
#include "gemm_wide.h"

// 8: buffer addressing, nontemporal stores; 9: 64-bit addresses and plain
// stores (row strides beyond 8 MiB, D columns not on 128-byte lines); 47:
// rows only 4-byte aligned, copied through registers.
#define TG_WIDE32_LIST(X)                          \
    X(8, TG_F32, 4, 5, 16, 1, 1, 5, 16, 96)            \
    X(9, TG_F32, 4, 5, 16, 0, 0, 0, 16, 93)            \
    X(47, TG_F32, 4, 4, 16, 1, 0, 18, 4, 88)

TG_WIDE32_LIST(TG_INSTANTIATE_WIDE)

#ifndef __HIP_DEVICE_COMPILE__
extern const TgKernelDesc tg_entries_wide32[] = {TG_WIDE32_LIST(TG_ENTRY_WIDE)};
extern const int tg_entries_wide32_count = sizeof(tg_entries_wide32) / sizeof(tg_entries_wide32[0]);
#endif  // __HIP_DEVICE_COMPILE__
