// Device helpers for the gfx950 tree-verify attention kernels: element types,
// bf16 conversion, wave reductions, MFMA wrappers, and the tree-mask builder.
#pragma once

#include "ta_common.h"

namespace ta {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- elements
// bf16 tensors are handled as their raw 16-bit patterns (uint16_t).
__device__ __forceinline__ float bf16_to_f32(uint16_t u) {
  return __builtin_bit_cast(float, static_cast<uint32_t>(u) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  // hardware conversion, round to nearest even
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

template <typename T> struct Elem;
template <> struct Elem<uint16_t> {
  static __device__ __forceinline__ float load_f(const uint16_t* p) { return bf16_to_f32(*p); }
  static __device__ __forceinline__ uint16_t from_f(float f) { return f32_to_bf16(f); }
};
template <> struct Elem<float> {
  static __device__ __forceinline__ float load_f(const float* p) { return *p; }
  static __device__ __forceinline__ float from_f(float f) { return f; }
};

// -------------------------------------------------------------- math
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Reductions over the four lanes l, l^16, l^32, l^48 (one MFMA output row).
// Exchange with lane l ^ 16 and with lane l ^ 32 on the VALU
// (v_permlane16_swap / v_permlane32_swap), no LDS round trip.  Called with
// the same value in both operands, the pair returned holds, in every lane,
// the lane's own value and its partner's (in an order that depends on the
// lane), so a symmetric reduction of the pair is the reduction over the two.
__device__ __forceinline__ float max_over_quads(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, v),
                                                  __builtin_bit_cast(unsigned, v), false, false);
  v = fmaxf(__builtin_bit_cast(float, unsigned(a[0])), __builtin_bit_cast(float, unsigned(a[1])));
  const auto b = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, v),
                                                  __builtin_bit_cast(unsigned, v), false, false);
  return fmaxf(__builtin_bit_cast(float, unsigned(b[0])), __builtin_bit_cast(float, unsigned(b[1])));
}
__device__ __forceinline__ float sum_over_quads(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, v),
                                                  __builtin_bit_cast(unsigned, v), false, false);
  v = __builtin_bit_cast(float, unsigned(a[0])) + __builtin_bit_cast(float, unsigned(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, v),
                                                  __builtin_bit_cast(unsigned, v), false, false);
  return __builtin_bit_cast(float, unsigned(b[0])) + __builtin_bit_cast(float, unsigned(b[1]));
}
// Integer sum, max and inclusive prefix sum over the 64 lanes of a wave, on
// the VALU with no LDS round trip: DPP steps within each row of 16 lanes
// (rotations by 8, 4, 2, 1 for the reductions, so every lane of a row ends
// with the row's result; shifts by 1, 2, 4, 8 for the prefix sum), then
// across rows the lane swaps l ^ 16 and l ^ 32 (reductions) or the row
// broadcasts of lanes 15 and 31 (prefix sum).  Every lane of the wave must be
// active.
constexpr int kDppRowShr = 0x110;    // + n: lane l of a row reads lane l - n (0 outside the row)
constexpr int kDppRowRor = 0x120;    // + n: lane l of a row reads lane (l - n) mod 16
constexpr int kDppRowBcast15 = 0x142;  // lane 15 of each row to the next row
constexpr int kDppRowBcast31 = 0x143;  // lane 31 to rows 2 and 3
__device__ __forceinline__ int wave_sum(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowRor + 8, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowRor + 4, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowRor + 2, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowRor + 1, 0xf, 0xf, false);
  const auto a = __builtin_amdgcn_permlane16_swap(unsigned(v), unsigned(v), false, false);
  v = int(a[0]) + int(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(unsigned(v), unsigned(v), false, false);
  return int(b[0]) + int(b[1]);
}
__device__ __forceinline__ int wave_max(int v) {
  v = max(v, __builtin_amdgcn_update_dpp(v, v, kDppRowRor + 8, 0xf, 0xf, false));
  v = max(v, __builtin_amdgcn_update_dpp(v, v, kDppRowRor + 4, 0xf, 0xf, false));
  v = max(v, __builtin_amdgcn_update_dpp(v, v, kDppRowRor + 2, 0xf, 0xf, false));
  v = max(v, __builtin_amdgcn_update_dpp(v, v, kDppRowRor + 1, 0xf, 0xf, false));
  const auto a = __builtin_amdgcn_permlane16_swap(unsigned(v), unsigned(v), false, false);
  v = max(int(a[0]), int(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(unsigned(v), unsigned(v), false, false);
  return max(int(b[0]), int(b[1]));
}
__device__ __forceinline__ int wave_inclusive_sum(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr + 1, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr + 2, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr + 4, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr + 8, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowBcast15, 0xa, 0xf, false);  // rows 1 and 3
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowBcast31, 0xc, 0xf, false);  // rows 2 and 3
  return v;
}

__device__ __forceinline__ void set_error(WsHeader* h, int code) {
  if (h) atomicCAS(&h->error, 0, code);
}

// ------------------------------------------------------------ tree mask
// One wave builds the ancestor-or-self words of one tree of T <= 64 nodes by
// pointer jumping: every lane i keeps the set of its ancestors within distance
// < 2^k and a link to its 2^k-th ancestor; one round ORs in the set held by that
// ancestor and follows its link, doubling the distance.  Six rounds reach any
// depth below 64.  Lanes >= T return 0.  `bad` is set (wave-uniformly) when a
// parent is neither -1 nor an earlier node; such a parent is treated as -1.
// [tree mask of the draft-token piece: pith.science review of arXiv
// 2508.08192, "What carries the argument"; ancestor-or-self as in SpecInfer]
// The same from parent values already in registers (lane i holds node i's
// parent; lanes >= T are ignored).
__device__ __forceinline__ uint64_t tree_mask_lanes(int p, int T, bool& bad) {
  const int lane = threadIdx.x & 63;
  int up = -1;
  bool lane_bad = false;
  if (lane < T) {
    lane_bad = !(p == -1 || (p >= 0 && p < lane));
    up = lane_bad ? -1 : p;
  }
  uint64_t anc = lane < T ? (uint64_t(1) << lane) : 0;
#pragma unroll
  for (int round = 0; round < 6; ++round) {
    const int src = up >= 0 ? up : lane;
    const uint32_t lo = __shfl(static_cast<uint32_t>(anc), src);
    const uint32_t hi = __shfl(static_cast<uint32_t>(anc >> 32), src);
    const int up2 = __shfl(up, src);
    if (up >= 0) {
      anc |= (static_cast<uint64_t>(hi) << 32) | lo;
      up = up2;
    }
  }
  bad = __any(lane_bad);
  return anc;
}

__device__ __forceinline__ uint64_t tree_mask_wave(const int32_t* parents, int T, bool& bad) {
  const int lane = threadIdx.x & 63;
  return tree_mask_lanes(lane < T ? parents[lane] : -1, T, bad);
}

}  // namespace ta
