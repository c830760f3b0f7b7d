// Device-side helpers shared by the attention kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace relattn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// Kernel arguments (one struct, passed by value).
struct AttnParams {
  const void* q;             // [T][H][D]
  const void* k;             // [num_blocks][bs][Hkv][D]
  const void* v;             // [num_blocks][bs][Hkv][D]
  const int32_t* block_table;  // [B][max_blocks]
  const int32_t* seqlens_k;  // [B]
  const int32_t* cu_q;       // [B+1]
  const void* rel;           // [T][H][E]
  void* out;                 // [T][H][D]
  float* ws_o;               // [splits][T][H][D]   (splits > 1)
  float* ws_lse;             // [splits][T][H]      (splits > 1)
  float* lse_out;            // [T][H] natural-log log-sum-exp of each row, or null (combine kernel)
  int T, B, max_q, max_blocks, H, Hkv, G, num_blocks, bs, E;
  float scale_log2;          // softmax_scale * log2(e)
  int causal, wl, wr, splits;
  int mode;                  // general kernel: 0 = every request, 1 = only S_b*G > 16
  int dec_chunk;             // decode kernel: keys per split (multiple of 16)
  int bs_log2;               // log2(block_size) when it is a power of two, else -1
  int kv_cap;                // keys a block-table row can address: min(max_blocks * bs, 2^31 - 1)
};

// s_waitcnt with only the vector-memory count constrained: wait until at
// most N vector memory operations of this wave are outstanding (they complete
// in issue order). gfx9 encoding: vmcnt bits [3:0] and [15:14], expcnt
// [6:4], lgkmcnt [11:8]; the other two fields are left at their maximum. The
// empty asm statements keep the compiler from moving memory accesses (LDS
// reads of the data being waited for) across the wait.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Two floats -> packed bf16 pair (round to nearest even, hardware convert).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2_t x = {lo, hi};
  bf16x2_t y = __builtin_convertvector(x, bf16x2_t);
  return __builtin_bit_cast(uint32_t, y);
}

// Reductions over the four lanes l, l^16, l^32, l^48 (same l%16) of a wave,
// with the gfx950 lane-swap instructions (VALU only, no LDS round trip):
// permlane32_swap on two copies of v yields v[l%32] and v[32 + l%32] in every
// lane, permlane16_swap likewise for the 16-lane rows.
__device__ __forceinline__ float wave_max_xor_16_32(float v) {
  const uint32_t u = __float_as_uint(v);
  auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t w = __float_as_uint(v);
  auto c = __builtin_amdgcn_permlane16_swap(w, w, false, false);
  return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}

__device__ __forceinline__ float wave_sum_xor_16_32(float v) {
  const uint32_t u = __float_as_uint(v);
  auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const uint32_t w = __float_as_uint(v);
  auto c = __builtin_amdgcn_permlane16_swap(w, w, false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// Physical row (in units of D elements) of logical key j of request b, KV head g.
__device__ __forceinline__ int64_t kv_row(const AttnParams& P, int b, int g, int j) {
  int page = P.block_table[(int64_t)b * P.max_blocks + j / P.bs];
  page = page < 0 ? 0 : (page >= P.num_blocks ? P.num_blocks - 1 : page);
  return ((int64_t)page * P.bs + (j % P.bs)) * P.Hkv + g;
}

// Request b's first packed row t0, query count S and key count L, clamped so
// that a malformed cu_seqlens_q / cache_seqlens can never index outside q,
// out, rel_logits or the request's block-table row. Returns false when the
// request has no rows.
__device__ __forceinline__ bool request_bounds(const AttnParams& P, int b, int& t0, int& S, int& L) {
  t0 = P.cu_q[b];
  const int t1 = P.cu_q[b + 1];
  if (t0 < 0 || t0 >= P.T || t1 <= t0) return false;
  S = min(t1, P.T) - t0;
  L = P.seqlens_k[b];
  L = L < 0 ? 0 : (L > P.kv_cap ? P.kv_cap : L);
  return true;
}

// Visible key range [lo, hi) of absolute query position p in a request of L keys.
__device__ __forceinline__ void visible_range(const AttnParams& P, int p, int L, int& lo, int& hi) {
  lo = 0;
  hi = L;
  if (P.causal) hi = min(hi, p + 1);
  if (P.wl >= 0) lo = max(lo, p - P.wl);
  if (P.wr >= 0) hi = min(hi, p + P.wr + 1);
  if (hi < lo) hi = lo;
}

}  // namespace relattn
