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

constexpr int kMaxSplits = 512;

// One workgroup of W waves per (token, head) row. The log-sum-exps are
// reduced over the whole workgroup; then each 16-byte load of a wave covers
// 64 / (D / 4) splits (D / 4 lanes per split, 4 dims per lane), the waves
// take interleaved groups of splits, and the per-lane sums are added across
// the split groups of a wave and across the waves through LDS.
template <bool BF16, int D, int W>
__global__ __launch_bounds__(W * 64) void combine_kernel(AttnParams P) {
  constexpr int kLanesPerSplit = D / 4;
  constexpr int kSplitsPerLoad = 64 / kLanesPerSplit;
  __shared__ float w_lds[kMaxSplits];
  __shared__ float red[W];
  __shared__ f32x4_t part[W][kSplitsPerLoad][kLanesPerSplit];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int64_t row = blockIdx.x;  // t * H + h
  const int64_t stride = (int64_t)P.T * P.H;  // between splits, in rows
  const int K = P.splits;

  // ---- weights exp(lse_k - LSE) ----
  float mx = kNegInf;
  for (int k = threadIdx.x; k < K; k += W * 64) {
    const float l = P.ws_lse[(int64_t)k * stride + row];
    w_lds[k] = l;
    mx = fmaxf(mx, l);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  mx = red[0];
#pragma unroll
  for (int w = 1; w < W; ++w) mx = fmaxf(mx, red[w]);
  __syncthreads();
  float sum = 0.f;
  if (mx != kNegInf) {
    for (int k = threadIdx.x; k < K; k += W * 64) {
      const float e = __expf(w_lds[k] - mx);
      w_lds[k] = e;
      sum += e;
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) sum += __shfl_xor(sum, o);
  if (lane == 0) red[wave] = sum;
  __syncthreads();
  sum = 0.f;
#pragma unroll
  for (int w = 0; w < W; ++w) sum += red[w];
  const float inv = sum > 0.f ? 1.f / sum : 0.f;
  if (P.lse_out != nullptr && threadIdx.x == 0) P.lse_out[row] = sum > 0.f ? mx + __logf(sum) : kNegInf;

  // ---- weighted sum of the partial outputs ----
  const int sub = lane / kLanesPerSplit;  // split within a load
  const int dl = lane % kLanesPerSplit;   // dims 4dl .. 4dl+3
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  if (mx != kNegInf) {
    constexpr int kStep = W * kSplitsPerLoad;
    int k = wave * kSplitsPerLoad + sub;
    // four loads in flight per lane
    for (; k + 3 * kStep < K; k += 4 * kStep) {
      f32x4_t v[4];
      float wk[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        wk[u] = w_lds[k + u * kStep];
        v[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if (wk[u] != 0.f)
          v[u] = *reinterpret_cast<const f32x4_t*>(P.ws_o + ((int64_t)(k + u * kStep) * stride + row) * D + 4 * dl);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) acc += wk[u] * v[u];
    }
    for (; k < K; k += kStep) {
      const float wk = w_lds[k];
      if (wk != 0.f)
        acc += wk * *reinterpret_cast<const f32x4_t*>(P.ws_o + ((int64_t)k * stride + row) * D + 4 * dl);
    }
  }
  part[wave][sub][dl] = acc;
  __syncthreads();
  if (wave == 0 && sub == 0) {
    f32x4_t r = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < W; ++w)
#pragma unroll
      for (int s = 0; s < kSplitsPerLoad; ++s) r += part[w][s][dl];
    r *= inv;
    if constexpr (BF16) {
      uint16_t* op = reinterpret_cast<uint16_t*>(P.out) + row * D + 4 * dl;
      *reinterpret_cast<u32x2_t*>(op) = u32x2_t{pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3])};
    } else {
      *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(P.out) + row * D + 4 * dl) = r;
    }
  }
}

template <bool BF16, int D>
int launch_rows(const AttnParams& P, int64_t rows, hipStream_t stream) {
  // enough waves per row that each handles about 16 splits
  constexpr int kSplitsPerLoad = 64 / (D / 4);
  const int per_wave = 8 * kSplitsPerLoad;
  const dim3 grid((unsigned)rows);
  if (P.splits <= per_wave) hipLaunchKernelGGL((combine_kernel<BF16, D, 1>), grid, dim3(64), 0, stream, P);
  else if (P.splits <= 4 * per_wave) hipLaunchKernelGGL((combine_kernel<BF16, D, 4>), grid, dim3(256), 0, stream, P);
  else hipLaunchKernelGGL((combine_kernel<BF16, D, 16>), grid, dim3(1024), 0, stream, P);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace

int launch_combine(const AttnParams& P, int dtype_bf16, int head_dim, hipStream_t stream) {
  const int64_t rows = (int64_t)P.T * P.H;
  if (rows == 0) return 0;
  if (P.splits > kMaxSplits || rows > 0x7fffffff) return -1;
  if (dtype_bf16) return head_dim == 128 ? launch_rows<true, 128>(P, rows, stream) : launch_rows<true, 64>(P, rows, stream);
  return head_dim == 128 ? launch_rows<false, 128>(P, rows, stream) : launch_rows<false, 64>(P, rows, stream);
}

}  // namespace relattn
