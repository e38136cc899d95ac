// ffn_lds.h -- internal: LDS layout of the hybrid-FFN GEMM launches (ffn.hip)
// and the host's choice of static LDS instance per launch.  Kept in a header
// that plain C++ also compiles, so that a CPU test can check, over the whole
// supported shape range, that every byte a launch touches lies inside the
// instance the host picks for it.
#pragma once

#if defined(__HIPCC__)
#define LR_FFN_HD __host__ __device__
#else
#define LR_FFN_HD
#endif

namespace lr {
namespace ffnlds {

constexpr int kWaves = 8;
constexpr int kRowPad = 16;                 // bytes of padding per token row of codes
constexpr int kLdsLimit = 160 * 1024;       // LDS of one gfx950 work-group

// One staged block of K columns: 16 token rows of codes (row stride K +
// kRowPad bytes), then the 16 x K/64 fp32 group scales.
LR_FFN_HD constexpr int row_stride(int k) { return k + kRowPad; }
LR_FFN_HD constexpr int scale_offset(int k) { return 16 * row_stride(k); }
LR_FFN_HD constexpr int block_bytes(int k) { return scale_offset(k) + 16 * (k / 64) * 4; }
// The wavefronts' partial tiles, [kWaves][RT][64 lanes] x 16 bytes, reuse the
// code area once the products are done; the reduced outputs (RT x 16 x 16
// fp32) follow the code area.  RT is at most 4 (the latent groups of
// k_ffn_in; pairs and the down projection take 2).
constexpr int kMaxRT = 4;
LR_FFN_HD constexpr int red_bytes(int rt) { return kWaves * rt * 64 * 16; }
LR_FFN_HD constexpr int code_area(int act) { return act > red_bytes(kMaxRT) ? act : red_bytes(kMaxRT); }
LR_FFN_HD constexpr int out_bytes(int rt) { return rt * 16 * 16 * 4; }
LR_FFN_HD constexpr int lds_bytes(int act) { return code_area(act) + out_bytes(kMaxRT); }

// Static instances: small (E <= 2048, r <= 1024, chunks of 2048), medium
// (E <= 4096, r <= 2048, chunks of 4096), large (E <= 8192, r <= 4096).
constexpr int kLdsS = lds_bytes(2 * block_bytes(1024));   // 39 424
constexpr int kLdsM = lds_bytes(2 * block_bytes(2048));   // 74 240
constexpr int kLdsL = lds_bytes(2 * block_bytes(4096));   // 143 872
static_assert(kLdsL <= kLdsLimit, "largest instance exceeds the LDS of a work-group");

// Bytes from the start of LDS up to the last one each launch touches.
LR_FFN_HD constexpr int in_extent(int E) { return code_area(block_bytes(E)) + out_bytes(4); }
LR_FFN_HD constexpr int mid_extent(int r) { return code_area(2 * block_bytes(r)) + out_bytes(2); }
LR_FFN_HD constexpr int out_extent(int kc, int rt) { return code_area(block_bytes(kc)) + out_bytes(rt); }

// The smallest instance that holds `need` bytes (0: none does).
inline int instance_for(int need) {
  return need <= kLdsS ? kLdsS : need <= kLdsM ? kLdsM : need <= kLdsL ? kLdsL : 0;
}

// Down projection: the hidden dimension (Fp, a multiple of 64) in chunks of
// 4096 (2048 for Fp <= 2048); with several chunks a work-group takes two row
// tiles of W_d, so each staged chunk of h serves 32 rows.
struct OutShape {
  int chunk, splits, rt, lds;
};
inline OutShape out_shape(int Fp) {
  OutShape s;
  s.chunk = Fp <= 2048 ? 2048 : 4096;
  s.splits = (Fp + s.chunk - 1) / s.chunk;
  s.rt = s.splits > 1 ? 2 : 1;
  s.lds = s.chunk == 2048 ? kLdsS : kLdsM;
  return s;
}

}  // namespace ffnlds
}  // namespace lr
