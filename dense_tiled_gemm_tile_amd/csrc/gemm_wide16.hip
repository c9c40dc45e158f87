// Wide streaming GEMM instances for bf16 and fp16 operands.
#include "gemm_wide.h"

// 0/1: the default for large products (nontemporal D stores, 16-bit D through
// the quad transpose); 2/3: plain stores, used when D columns do not start on
// 128-byte lines (nontemporal stores of the partial lines at the tile edges
// measured about 20 % slower), fp32 D through the LDS transpose; 4/5: 64-bit
// addresses for row strides beyond 8 MiB; 6/7: with the softmax epilogue;
// 43-46: operand rows only 4- or 2-byte aligned, copied through registers
// (43/44 with the nontemporal-store epilogue of 0/1, 45/46 with the
// plain-store one of 2/3); their weight is the measured ratio to the aligned
// kernel on 12289x5003x4099 bf16 (0.52 ms against 0.42 ms on the staged
// copies, settled clock): 107 x 0.80.
#define TG_WIDE16_LIST(X)                          \
    X(0, TG_BF16, 4, 5, 16, 1, 1, 17, 16, 107)         \
    X(1, TG_F16, 4, 5, 16, 1, 1, 17, 16, 107)          \
    X(2, TG_BF16, 4, 5, 16, 1, 1, 18, 16, 107)         \
    X(3, TG_F16, 4, 5, 16, 1, 1, 18, 16, 107)          \
    X(4, TG_BF16, 4, 5, 16, 0, 0, 0, 16, 105)          \
    X(5, TG_F16, 4, 5, 16, 0, 0, 0, 16, 105)           \
    X(6, TG_BF16, 4, 5, 16, 1, 1, 13, 16, 106)         \
    X(7, TG_F16, 4, 5, 16, 1, 1, 13, 16, 106)          \
    X(43, TG_BF16, 4, 4, 16, 1, 0, 17, 2, 85)          \
    X(44, TG_F16, 4, 4, 16, 1, 0, 17, 2, 85)           \
    X(45, TG_BF16, 4, 4, 16, 1, 0, 18, 2, 85)          \
    X(46, TG_F16, 4, 4, 16, 1, 0, 18, 2, 85)

TG_WIDE16_LIST(TG_INSTANTIATE_WIDE)

#ifndef __HIP_DEVICE_COMPILE__
extern const TgKernelDesc tg_entries_wide16[] = {TG_WIDE16_LIST(TG_ENTRY_WIDE)};
extern const int tg_entries_wide16_count = sizeof(tg_entries_wide16) / sizeof(tg_entries_wide16[0]);
#endif  // __HIP_DEVICE_COMPILE__
