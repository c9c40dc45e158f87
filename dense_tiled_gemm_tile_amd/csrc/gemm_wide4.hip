// Wide streaming GEMM instances for 4-bit (e2m1) operands on the 32x32x64
// scaled MFMA.  One 16-byte chunk of a row is one MFMA fragment (32 k), so
// these run the 16-bit schedule unchanged: a stage is 128 bytes (256 k) per
// row, four slabs of 16 MFMAs.  51: nontemporal D stores; 52: plain stores
// (D columns not on 128-byte lines); 53: operand rows only 4-, 2- or 1-byte
// aligned, copied through registers; 54/55: with block scales (four-slot
// schedule, the scales in the fifth slot), nontemporal and plain stores;
// 56: 64-bit addresses for row strides beyond 8 MiB (K above 2^24).
#include "gemm_wide.h"

#define TG_WIDE4_LIST(X)                           \
    X(51, TG_E2M1, 4, 5, 16, 1, 1, 17, 16, 107)        \
    X(52, TG_E2M1, 4, 5, 16, 1, 1, 18, 16, 107)        \
    X(53, TG_E2M1, 4, 4, 16, 1, 0, 18, 1, 95)          \
    X(54, TG_E2M1, 4, 4, 16, 1, 0, 81, 16, 100)        \
    X(55, TG_E2M1, 4, 4, 16, 1, 0, 82, 16, 100)        \
    X(56, TG_E2M1, 4, 5, 16, 0, 0, 0, 16, 105)

TG_WIDE4_LIST(TG_INSTANTIATE_WIDE)

#ifndef __HIP_DEVICE_COMPILE__
extern const TgKernelDesc tg_entries_wide4[] = {TG_WIDE4_LIST(TG_ENTRY_WIDE)};
extern const int tg_entries_wide4_count = sizeof(tg_entries_wide4) / sizeof(tg_entries_wide4[0]);
#endif  // __HIP_DEVICE_COMPILE__
