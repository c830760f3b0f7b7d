// Split-KV merge: each split wrote its normalised partial output o_k and its
// log-sum-exp lse_k for every (token, head); the result is
//   out = sum_k exp(lse_k - LSE) o_k,  LSE = log sum_k exp(lse_k),
// with empty splits (lse_k = -inf) contributing nothing and an all-empty row
// giving zeros. This is the num_splits / split-KV combine of the
// docs.vllm.ai inkling_fa4_num_splits and inkling_fa4_rel_attention pages.
#include "device_common.h"
#include "kernels.h"

namespace relattn {

namespace {

// One wave per (token, head); lanes own head_dim / 64 consecutive dims.
// Lane l reads the log-sum-exps of splits l, l+64, ... (up to kMaxPerLane
// of them, so at most 64 * kMaxPerLane splits).
constexpr int kMaxPerLane = 8;

template <bool BF16, int D>
__global__ __launch_bounds__(256) void combine_kernel(AttnParams P) {
  __shared__ float w_lds[4][64 * kMaxPerLane];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + wave;  // t * H + h
  const int64_t nrows = (int64_t)P.T * P.H;
  if (row >= nrows) return;
  const int64_t stride = nrows;  // between splits, in rows
  const int K = P.splits;

  float l[kMaxPerLane];
  float mx = kNegInf;
#pragma unroll
  for (int e = 0; e < kMaxPerLane; ++e) {
    const int k = lane + 64 * e;
    l[e] = k < K ? P.ws_lse[(int64_t)k * stride + row] : kNegInf;
    mx = fmaxf(mx, l[e]);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  constexpr int kPer = D / 64;
  float acc[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) acc[e] = 0.f;
  if (mx != kNegInf) {
    float sum = 0.f;
#pragma unroll
    for (int e = 0; e < kMaxPerLane; ++e) {
      l[e] = __expf(l[e] - mx);
      sum += l[e];
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) sum += __shfl_xor(sum, o);
    const float inv = 1.f / sum;
#pragma unroll
    for (int e = 0; e < kMaxPerLane; ++e) w_lds[wave][lane + 64 * e] = l[e] * inv;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    for (int k = 0; k < K; ++k) {
      const float w = w_lds[wave][k];
      if (w == 0.f) continue;
      const float* src = P.ws_o + ((int64_t)k * stride + row) * D + lane * kPer;
#pragma unroll
      for (int e = 0; e < kPer; ++e) acc[e] = fmaf(w, src[e], acc[e]);
    }
  }
  if constexpr (BF16) {
    uint16_t* op = reinterpret_cast<uint16_t*>(P.out) + row * D + lane * kPer;
    if constexpr (kPer == 2) {
      *reinterpret_cast<uint32_t*>(op) = pack_bf16x2(acc[0], acc[1]);
    } else {
      op[0] = (uint16_t)(pack_bf16x2(acc[0], 0.f) & 0xffffu);
    }
  } else {
    float* op = reinterpret_cast<float*>(P.out) + row * D + lane * kPer;
#pragma unroll
    for (int e = 0; e < kPer; ++e) op[e] = acc[e];
  }
}

}  // namespace

int launch_combine(const AttnParams& P, int dtype_bf16, int head_dim, hipStream_t stream) {
  const int64_t rows = (int64_t)P.T * P.H;
  if (rows == 0) return 0;
  if (P.splits > 64 * kMaxPerLane) return -1;
  dim3 grid((unsigned)((rows + 3) / 4));
  dim3 block(256);
  if (dtype_bf16) {
    if (head_dim == 128) hipLaunchKernelGGL((combine_kernel<true, 128>), grid, block, 0, stream, P);
    else hipLaunchKernelGGL((combine_kernel<true, 64>), grid, block, 0, stream, P);
  } else {
    if (head_dim == 128) hipLaunchKernelGGL((combine_kernel<false, 128>), grid, block, 0, stream, P);
    else hipLaunchKernelGGL((combine_kernel<false, 64>), grid, block, 0, stream, P);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace relattn
