// Gate MLP score of every token (TokenGate article, section "How does
// TokenGate learned token pruning work?": an MLP scores each token from its
// post-attention residual at the gate layer):
//     s_t = b2 + sum_f w2[f] * SiLU(b1[f] + W1[f, :] . hidden[t, :])
//
// bf16 path: one workgroup of 2 * F/64 waves scores 256 tokens.  The product
// is computed transposed, C^T[f][t] = W1[f] . h[t], with the 32x32x16 bf16
// MFMA, so that each lane of the accumulator holds one token's column and a
// run of F rows: the SiLU . w2 epilogue then reduces over F inside the lane,
// across the two wave halves, and across the F-quarter waves through LDS, in
// a fixed order (bit-reproducible, no atomics).  The [T, F] activation never
// reaches memory.  hidden and W1 stream through one LDS stage of 64 columns
// with register prefetch of the next stage.
#include "tg_common.h"

namespace tg {
namespace {

constexpr int kGateBM = 256;  // tokens per workgroup
constexpr int kGateBK = 64;   // reduction columns per LDS stage
constexpr int kRowChunks = kGateBK / 8;  // 16-byte chunks per staged row

// XOR swizzle of the 16-byte chunk inside a 128-byte staged row: rows r and
// r + 1 share a 256-byte bank window, so (r & 1, chunk ^ ((r >> 1) & 7)) is
// distinct over any 16 consecutive rows and a fragment read of 32 rows at
// one logical chunk touches every bank twice at most.
__device__ __forceinline__ int swz_chunk(int row, int c) { return c ^ ((row >> 1) & 7); }

template <int NFQ>  // number of 64-wide F quarters (F = 64 * NFQ)
__global__ __launch_bounds__(128 * NFQ) void gate_bf16_kernel(
    const uint16_t* __restrict__ hidden, int64_t ld, int64_t T, int D,
    const uint16_t* __restrict__ W1, const float* __restrict__ b1,
    const float* __restrict__ w2, float b2, float* __restrict__ scores) {
  constexpr int F = 64 * NFQ;
  constexpr int NT = 128 * NFQ;                    // threads
  constexpr int H_CHUNKS = kGateBM * kRowChunks;   // 2048 chunks of hidden
  constexpr int W_CHUNKS = F * kRowChunks;
  constexpr int H_PER_T = H_CHUNKS / NT;
  constexpr int W_PER_T = W_CHUNKS / NT;
  static_assert(H_CHUNKS % NT == 0 && W_CHUNKS % NT == 0, "tile split");

  __shared__ uint4 sh_h[kGateBM * kRowChunks];
  __shared__ uint4 sh_w[F * kRowChunks];
  __shared__ float sh_red[NFQ][kGateBM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wt = wave / NFQ;  // token half: tokens [128 wt, 128 wt + 128)
  const int wf = wave % NFQ;  // F quarter: rows [64 wf, 64 wf + 64)
  const int64_t t0 = (int64_t)blockIdx.x * kGateBM;

  uint4 pre_h[H_PER_T];
  uint4 pre_w[W_PER_T];

  auto prefetch = [&](int kc) {
    const int k0 = kc * kGateBK;
#pragma unroll
    for (int j = 0; j < H_PER_T; ++j) {
      const int id = tid + j * NT;
      const int r = id / kRowChunks, c = id % kRowChunks;
      const int64_t t = t0 + r;
      if (t < T)
        pre_h[j] = *reinterpret_cast<const uint4*>(hidden + t * ld + k0 + c * 8);
      else
        pre_h[j] = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < W_PER_T; ++j) {
      const int id = tid + j * NT;
      const int r = id / kRowChunks, c = id % kRowChunks;
      pre_w[j] = *reinterpret_cast<const uint4*>(W1 + (int64_t)r * D + k0 + c * 8);
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int j = 0; j < H_PER_T; ++j) {
      const int id = tid + j * NT;
      const int r = id / kRowChunks, c = id % kRowChunks;
      sh_h[r * kRowChunks + swz_chunk(r, c)] = pre_h[j];
    }
#pragma unroll
    for (int j = 0; j < W_PER_T; ++j) {
      const int id = tid + j * NT;
      const int r = id / kRowChunks, c = id % kRowChunks;
      sh_w[r * kRowChunks + swz_chunk(r, c)] = pre_w[j];
    }
  };

  f32x16 acc[2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.0f;

  const int nk = D / kGateBK;
  prefetch(0);
  for (int kc = 0; kc < nk; ++kc) {
    __syncthreads();
    stage();
    __syncthreads();
    if (kc + 1 < nk) prefetch(kc + 1);
#pragma unroll
    for (int ks = 0; ks < kGateBK / 16; ++ks) {
      const int c = ks * 2 + (lane >> 5);
      bf16x8 fa[2], fb[4];
#pragma unroll
      for (int fbk = 0; fbk < 2; ++fbk) {
        const int r = wf * 64 + fbk * 32 + (lane & 31);
        fa[fbk] = as_bf16x8(sh_w[r * kRowChunks + swz_chunk(r, c)]);
      }
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        const int r = wt * 128 + tb * 32 + (lane & 31);
        fb[tb] = as_bf16x8(sh_h[r * kRowChunks + swz_chunk(r, c)]);
      }
#pragma unroll
      for (int fbk = 0; fbk < 2; ++fbk)
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) acc[fbk][tb] = mfma32x32x16(fa[fbk], fb[tb], acc[fbk][tb]);
    }
  }

  // Epilogue: lane holds token column (lane & 31) of each token block and F
  // rows acc_row(i, lane) of each F block.
  float bb[2][16], ww[2][16];
#pragma unroll
  for (int fbk = 0; fbk < 2; ++fbk)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int f = wf * 64 + fbk * 32 + acc_row(i, lane);
      bb[fbk][i] = b1 ? b1[f] : 0.0f;
      ww[fbk][i] = w2[f];
    }
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) {
    float part = 0.0f;
#pragma unroll
    for (int fbk = 0; fbk < 2; ++fbk)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float a = acc[fbk][tb][i] + bb[fbk][i];
        const float z = a / (1.0f + __expf(-a));
        part = fmaf(ww[fbk][i], z, part);
      }
    part = pair_sum(part);
    if (lane < 32) sh_red[wf][wt * 128 + tb * 32 + lane] = part;
  }
  __syncthreads();
  for (int r = tid; r < kGateBM; r += NT) {
    const int64_t t = t0 + r;
    if (t < T) {
      float s = 0.0f;
#pragma unroll
      for (int q = 0; q < NFQ; ++q) s += sh_red[q][r];
      scores[t] = s + b2;
    }
  }
}

// fp32 path: one wave per token, lanes split F; the dot products over D run
// sequentially in fp32, the F reduction is a fixed shuffle tree.
__global__ __launch_bounds__(256) void gate_f32_kernel(
    const float* __restrict__ hidden, int64_t ld, int64_t T, int D,
    const float* __restrict__ W1, const float* __restrict__ b1,
    const float* __restrict__ w2, float b2, int F, float* __restrict__ scores) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* h = hidden + t * ld;
  float part = 0.0f;
  for (int f = lane; f < F; f += 64) {
    const float* w = W1 + (int64_t)f * D;
    float a = b1 ? b1[f] : 0.0f;
    for (int k = 0; k < D; ++k) a = fmaf(w[k], h[k], a);
    const float z = a / (1.0f + __expf(-a));
    part = fmaf(w2[f], z, part);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off);
  if (lane == 0) scores[t] = part + b2;
}

}  // namespace

hipError_t launch_gate_bf16(const void* hidden, int64_t ld, int64_t T, int D, const void* W1,
                            const float* b1, const float* w2, float b2, int F, float* scores,
                            hipStream_t s) {
  if (T == 0) return hipSuccess;
  const dim3 grid((unsigned)((T + kGateBM - 1) / kGateBM));
  const auto* h = static_cast<const uint16_t*>(hidden);
  const auto* w = static_cast<const uint16_t*>(W1);
  switch (F) {
    case 64: hipLaunchKernelGGL(gate_bf16_kernel<1>, grid, dim3(128), 0, s, h, ld, T, D, w, b1, w2, b2, scores); break;
    case 128: hipLaunchKernelGGL(gate_bf16_kernel<2>, grid, dim3(256), 0, s, h, ld, T, D, w, b1, w2, b2, scores); break;
    case 256: hipLaunchKernelGGL(gate_bf16_kernel<4>, grid, dim3(512), 0, s, h, ld, T, D, w, b1, w2, b2, scores); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gate_f32(const float* hidden, int64_t ld, int64_t T, int D, const float* W1,
                           const float* b1, const float* w2, float b2, int F, float* scores,
                           hipStream_t s) {
  if (T == 0) return hipSuccess;
  const dim3 grid((unsigned)((T + 3) / 4));
  hipLaunchKernelGGL(gate_f32_kernel, grid, dim3(256), 0, s, hidden, ld, T, D, W1, b1, w2, b2, F,
                     scores);
  return hipGetLastError();
}

}  // namespace tg
