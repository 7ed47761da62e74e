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
// reaches memory.  hidden and W1 stream through four LDS stages of 32
// columns, filled by buffer-to-LDS loads (no registers in between) issued
// three stages ahead of the MFMAs that read them.
#include "tg_common.h"

namespace tg {
namespace {

constexpr int kGateBM = 256;  // tokens per workgroup
constexpr int kGateBK = 32;   // reduction columns per LDS stage
constexpr int kGateStages = 4;
constexpr int kBufFlags = 0x00020000;  // raw buffer: reads past num_records give 0

// Stage layout: a row of 32 bf16 columns is four 16-byte chunks, rows are
// packed (64 bytes), and chunk c of row r sits at position c ^ ((r >> 2) & 3)
// so that a fragment read of 16 consecutive rows at one column touches 16
// different bank groups.
__device__ __forceinline__ int gate_swz(int r, int c) { return c ^ ((r >> 2) & 3); }

template <int NFQ>  // number of 64-wide F quarters (F = 64 * NFQ)
__global__ __launch_bounds__(128 * NFQ) void gate_bf16_kernel(
    const uint16_t* __restrict__ hidden, int64_t ld, int64_t T, int D,
    const uint16_t* __restrict__ W1, const float* __restrict__ b1,
    const float* __restrict__ w2, float b2, float* __restrict__ scores) {
  constexpr int F = 64 * NFQ;
  constexpr int NT = 128 * NFQ;              // threads
  constexpr int NW = NT / 64;                // waves
  constexpr int ROW_B = kGateBK * 2;         // bytes per staged row
  constexpr int H_BYTES = kGateBM * ROW_B;   // hidden stage
  constexpr int W_BYTES = F * ROW_B;         // W1 stage
  constexpr int H_DMA = H_BYTES / 1024 / NW; // 1 KB wave copies per wave per stage
  constexpr int W_DMA = W_BYTES / 1024 / NW;
  constexpr int ND = H_DMA + W_DMA;          // global loads per thread per stage
  static_assert(H_BYTES % (1024 * NW) == 0 && W_BYTES % (1024 * NW) == 0, "stage split");

  // Four stages, each its own array so that the compiler can tell the stage
  // being loaded from the ones being read.
  __shared__ __attribute__((aligned(16))) char sh_h0[H_BYTES], sh_h1[H_BYTES], sh_h2[H_BYTES], sh_h3[H_BYTES];
  __shared__ __attribute__((aligned(16))) char sh_w0[W_BYTES], sh_w1[W_BYTES], sh_w2[W_BYTES], sh_w3[W_BYTES];
  __shared__ float sh_red[NFQ][kGateBM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wt = wave / NFQ;  // token half: tokens [128 wt, 128 wt + 128)
  const int wf = wave % NFQ;  // F quarter: rows [64 wf, 64 wf + 64)
  const int64_t t0 = (int64_t)blockIdx.x * kGateBM;
  const int rows = (int)min((int64_t)kGateBM, T - t0);
  const uint16_t* hbase = hidden + t0 * ld;

  // Per-thread source offsets of its 16 bytes in each wave copy: copy j of
  // this wave covers rows 16 (wave * COPIES + j) .. +15; lane l writes
  // position l % 4 of row l / 4, which holds the row's chunk
  // (l % 4) ^ ((row >> 2) & 3).
  int h_src[H_DMA], w_src[W_DMA];
#pragma unroll
  for (int j = 0; j < H_DMA; ++j) {
    const int r = (wave * H_DMA + j) * 16 + (lane >> 2);
    h_src[j] = (r * (int)ld + gate_swz(r, lane & 3) * 8) * 2;
  }
#pragma unroll
  for (int j = 0; j < W_DMA; ++j) {
    const int r = (wave * W_DMA + j) * 16 + (lane >> 2);
    w_src[j] = (r * D + gate_swz(r, lane & 3) * 8) * 2;
  }
  // Buffer-to-LDS loads of reduction columns [k0, k0 + 32) into one stage;
  // hidden rows past T, and columns past D, read as zero (the descriptor's
  // range check also keeps every access inside the two arrays).  The loads
  // are written as instructions of their own so that the compiler does not
  // wait for them at the next LDS read: their completion is waited for
  // explicitly, two stages later, before the barrier that precedes the
  // first read of their stage.
  auto dma = [&](const uint16_t* base, int bytes, char* lds, int voff) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, bytes, kBufFlags);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, 0, 0, 0);
  };
  auto load_stage = [&](int k0, char* sh, char* sw) __attribute__((always_inline)) {
    const int kk = __builtin_amdgcn_readfirstlane(min(k0, D));
    const int hb = __builtin_amdgcn_readfirstlane(k0 < D ? rows * (int)ld * 2 - kk * 2 : 0);
    const int wb = __builtin_amdgcn_readfirstlane(k0 < D ? F * D * 2 - kk * 2 : 0);
#pragma unroll
    for (int j = 0; j < H_DMA; ++j) dma(hbase + kk, hb, sh + (wave * H_DMA + j) * 1024, h_src[j]);
#pragma unroll
    for (int j = 0; j < W_DMA; ++j) dma(W1 + kk, wb, sw + (wave * W_DMA + j) * 1024, w_src[j]);
  };

  f32x16 acc[2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.0f;

  // MFMAs over one stage: two k-steps of 16 columns.  Every fragment row
  // is a multiple of 32 plus lane % 32, so its swizzle term is
  // (lane >> 2) & 3 and the per-lane part of the address depends on the
  // k-step only; rows of different fragments differ by constants.
  int a_off[kGateBK / 16], b_off[kGateBK / 16];
#pragma unroll
  for (int ks = 0; ks < kGateBK / 16; ++ks) {
    const int lane_part = (lane & 31) * ROW_B + (((ks * 2 + (lane >> 5)) ^ ((lane >> 2) & 3)) * 16);
    a_off[ks] = wf * 64 * ROW_B + lane_part;
    b_off[ks] = wt * 128 * ROW_B + lane_part;
  }
  auto compute_stage = [&](const char* sh, const char* sw) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < kGateBK / 16; ++ks) {
      bf16x8 fa[2], fb[4];
#pragma unroll
      for (int fbk = 0; fbk < 2; ++fbk)
        fa[fbk] = *reinterpret_cast<const bf16x8*>(sw + a_off[ks] + fbk * 32 * ROW_B);
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
        fb[tb] = *reinterpret_cast<const bf16x8*>(sh + b_off[ks] + tb * 32 * ROW_B);
#pragma unroll
      for (int fbk = 0; fbk < 2; ++fbk)
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) acc[fbk][tb] = mfma32x32x16(fa[fbk], fb[tb], acc[fbk][tb]);
    }
  };
  // End of a stage: this wave's loads of the stage two steps back are
  // complete (ND loads are issued per stage and complete in order) and its
  // LDS reads are done; then all waves meet.  An LDS-only barrier: the
  // loads of the newer stages stay in flight across it.
#define TG_GATE_SYNC() asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(2 * ND) : "memory")

  // Stage s holds reduction columns [32 k, 32 k + 32) for k = s mod 4; the
  // loads of k + 3 are issued while k is computed.  The step count is
  // rounded up to a multiple of four: steps past D load zeros (an
  // out-of-range buffer-to-LDS load writes zeros) and add nothing.
  const int nk = (D / kGateBK + 3) & ~3;
  load_stage(0, sh_h0, sh_w0);
  load_stage(kGateBK, sh_h1, sh_w1);
  load_stage(2 * kGateBK, sh_h2, sh_w2);
  TG_GATE_SYNC();
  for (int k = 0; k < nk; k += 4) {
    load_stage((k + 3) * kGateBK, sh_h3, sh_w3);
    compute_stage(sh_h0, sh_w0);
    TG_GATE_SYNC();
    load_stage((k + 4) * kGateBK, sh_h0, sh_w0);
    compute_stage(sh_h1, sh_w1);
    TG_GATE_SYNC();
    load_stage((k + 5) * kGateBK, sh_h1, sh_w1);
    compute_stage(sh_h2, sh_w2);
    TG_GATE_SYNC();
    load_stage((k + 6) * kGateBK, sh_h2, sh_w2);
    compute_stage(sh_h3, sh_w3);
    TG_GATE_SYNC();
  }
#undef TG_GATE_SYNC
  // the trailing loads (past D) must land before the workgroup's LDS is released
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

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
      float sum = 0.0f;
#pragma unroll
      for (int q = 0; q < NFQ; ++q) sum += sh_red[q][r];
      scores[t] = sum + b2;
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
