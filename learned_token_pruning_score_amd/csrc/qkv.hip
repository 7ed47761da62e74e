// Attention inputs of the pruned layers: the fused q/k/v projection of the
// kept rows with the rotary position embedding at their original positions.
//
// TokenGate article, section "How does TokenGate learned token pruning
// work?": the layers above the gate run on the kept tokens only, and each
// kept token keeps the position id it had in the full prompt.  With
// W_qkv [(Hq + 2 Hkv) d, D] (rows: the q heads, then the k heads, then the
// v heads) and the rotary embedding of the Qwen3 family in the rotate-half
// form (element i of a head pairs with element i + d/2, angle
// pos * theta^(-2 i / d)):
//     y_t   = W_qkv . x_t
//     q, k: (y_i, y_{i+d/2}) <- (y_i c - y_{i+d/2} s,  y_{i+d/2} c + y_i s)
//     v:    unchanged
//
// Two kernels:
//   rope_table  cos / sin of every (kept row, frequency) pair, evaluated in
//               fp64 from the row's position and stored as fp32 pairs
//               [Kt, d/2].  It depends on the positions only, so a pruned
//               forward builds it once and every layer reuses it.
//   qkv_rope    bf16: C^T[n][t] = W_qkv[n] . x[t] on the 32x32x16 bf16 MFMA,
//               the same pipeline as the gate MLP (rows of x straight from
//               HBM into the registers that serve as the B operand, three
//               64-column stages ahead; W_qkv through four LDS stages filled
//               by buffer-to-LDS loads).  A workgroup of 8 waves owns tiles
//               of 256 rows x 256 output columns, each wave 32 rows.  Head
//               boundaries fall on tile boundaries (d divides 256), and the
//               32-column blocks j and j + d/64 of a head hold the two halves
//               of a rotation pair in the same lane and register, so the
//               rotation happens in registers before the bf16 store.
//               fp32: one thread per output, dot products on vector ALUs.

#include "tg_common.h"

namespace tg {
namespace {

constexpr int kQkvBK = 64;    // reduction columns per stage (128-byte row segments)
constexpr int kQkvAhead = 3;  // stages loaded ahead of the one computed
constexpr int kQkvBM = 256;   // rows of x per tile (8 waves x 32)
constexpr int kQkvBN = 256;   // output columns per tile
constexpr int kQkvNFB = kQkvBN / 32;
constexpr int kBufFlags = 0x00020000;  // raw buffer: reads past num_records give 0

// A staged row of W_qkv is 64 columns = eight 16-byte chunks; logical chunk
// c of row r sits at position c ^ ((r >> 1) & 7), so that the fragment
// reads of 16 consecutive rows at one chunk touch 16 different bank groups.
__device__ __forceinline__ int qkv_swz(int r, int c) { return c ^ ((r >> 1) & 7); }

// One 16-byte buffer-to-LDS load per lane: lane l writes bytes
// [16 l, 16 l + 16) of lds.  Out-of-range reads write zeros.
__device__ __forceinline__ void qkv_lds_load16(__amdgpu_buffer_rsrc_t r, char* lds, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, 0, 0, 0);
}

__global__ __launch_bounds__(256) void rope_table_kernel(const int32_t* __restrict__ pos, int64_t n,
                                                         int d, double theta, float2* __restrict__ table) {
  const int half = d / 2;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= n * half) return;
  const int64_t t = idx / half;
  const int i = (int)(idx - t * half);
  const double inv_freq = pow(theta, -2.0 * (double)i / (double)d);
  const double ang = (double)pos[t] * inv_freq;
  double s, c;
  sincos(ang, &s, &c);
  table[idx] = make_float2((float)c, (float)s);
}

// Reduction order inside a stage: a lane of half h = lane / 32 supplies, for
// k-step j, the 8 columns [32 h + 8 j, 32 h + 8 j + 8) of its stage, for x
// and for the W_qkv fragments alike, so the products sum over the columns of
// the definition, in another order.
template <int HD>
__global__ __launch_bounds__(512, 1) void qkv_rope_bf16_kernel(
    const uint16_t* __restrict__ x, int64_t ld, int64_t Kt, int D,
    const uint16_t* __restrict__ W, int N, int rot_cols, int n_nt, int n_tiles,
    const float2* __restrict__ rope, uint16_t* __restrict__ out, int64_t ld_out) {
  constexpr int NW = 8;
  constexpr int W_BYTES = kQkvBN * kQkvBK * 2;  // one stage of W_qkv
  constexpr int W_DMA = W_BYTES / 1024 / NW;   // 1 KB buffer-to-LDS copies per wave per stage
  constexpr int PER = W_DMA + 4;               // vector-memory instructions per wave per stage
  constexpr int BPH = HD / 32;                 // 32-column blocks per head
  constexpr int P = BPH / 2;                   // distance from a block to its rotation partner
  static_assert(W_BYTES % (1024 * NW) == 0, "stage split");
  static_assert(kQkvBN % HD == 0, "heads must not straddle tiles");

  __shared__ __attribute__((aligned(16))) char sw0[W_BYTES], sw1[W_BYTES], sw2[W_BYTES], sw3[W_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // Stages per tile, rounded up to a multiple of four (the unroll below);
  // stages past D load zeros and add nothing.
  const int nk = (D / kQkvBK + 3) & ~3;
  const int my_tiles = ((int)blockIdx.x < n_tiles) ? (n_tiles - 1 - (int)blockIdx.x) / (int)gridDim.x + 1 : 0;
  const int n_steps = my_tiles * nk;

  // x: lane loads 64 contiguous bytes of row 32 wave + lane % 32 of the tile
  const int h_voff = ((wave * 32 + (lane & 31)) * (int)ld + (lane >> 5) * 32) * 2;
  // W_qkv copies: copy j of this wave fills rows 8 (wave * W_DMA + j) .. +7;
  // lane l writes position l % 8 of row l / 8, which holds that row's
  // logical chunk qkv_swz(row, l % 8).
  int w_src[W_DMA];
#pragma unroll
  for (int j = 0; j < W_DMA; ++j) {
    const int r = (wave * W_DMA + j) * 8 + (lane >> 3);
    w_src[j] = (r * D + qkv_swz(r, lane & 7) * 8) * 2;
  }
  // W_qkv fragment of column block fb, k-step ks: row 32 fb + lane % 32,
  // logical chunk 4 (lane / 32) + ks; the swizzle term depends on the lane.
  int a_off[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    a_off[ks] = (lane & 31) * (kQkvBK * 2) + qkv_swz(lane & 31, 4 * (lane >> 5) + ks) * 16;

  // Load position: tile ld_tile (a multiple of gridDim.x past blockIdx.x),
  // stage ld_k of it; tile id = row tile * n_nt + column tile.  Loads past
  // the last tile read nothing (zero range).
  int ld_tile = blockIdx.x, ld_k = 0;
  int ld_mt = ld_tile / n_nt, ld_nt = ld_tile - ld_mt * n_nt;
  auto issue = [&](char* sw, uint4 (&h)[4]) __attribute__((always_inline)) {
    const bool tin = ld_tile < n_tiles;
    const int64_t t0 = (int64_t)ld_mt * kQkvBM;
    const int c0 = ld_nt * kQkvBN;
    const int rows = tin ? (int)min((int64_t)kQkvBM, Kt - t0) : 0;
    const int cols = tin ? min(kQkvBN, N - c0) : 0;
    const int k0 = ld_k * kQkvBK;
    const bool kin = k0 < D;
    const int kk = kin ? k0 : 0;
    const int hb = __builtin_amdgcn_readfirstlane((rows > 0 && kin) ? rows * (int)ld * 2 - kk * 2 : 0);
    const int wb = __builtin_amdgcn_readfirstlane((cols > 0 && kin) ? cols * D * 2 - kk * 2 : 0);
    const uint16_t* hb_ptr = rows > 0 ? x + t0 * ld + kk : x;
    const uint16_t* wb_ptr = cols > 0 ? W + (int64_t)c0 * D + kk : W;
    const __amdgpu_buffer_rsrc_t rh = __builtin_amdgcn_make_buffer_rsrc((void*)hb_ptr, (short)0, hb, kBufFlags);
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc((void*)wb_ptr, (short)0, wb, kBufFlags);
#pragma unroll
    for (int j = 0; j < W_DMA; ++j)
      qkv_lds_load16(rw, sw + (wave * W_DMA + j) * 1024, w_src[j]);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      h[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rh, h_voff + 16 * j, 0, 0));
    if (++ld_k == nk) {
      ld_k = 0;
      ld_tile += gridDim.x;
      ld_mt = ld_tile / n_nt;
      ld_nt = ld_tile - ld_mt * n_nt;
    }
  };

  f32x16 acc[kQkvNFB];
#pragma unroll
  for (int fb = 0; fb < kQkvNFB; ++fb)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[fb][i] = 0.0f;

  // One stage: 4 k-steps x 8 column blocks; each W_qkv fragment is read
  // three MFMAs ahead of its use.
  constexpr int NM = 4 * kQkvNFB;
  constexpr int AHEAD = 3;
  auto compute = [&](const char* sw, const uint4 (&h)[4]) __attribute__((always_inline)) {
    bf16x8 fa[NM];
    auto frag = [&](int m) __attribute__((always_inline)) {
      const int ks = m / kQkvNFB, fb = m % kQkvNFB;
      return *reinterpret_cast<const bf16x8*>(sw + a_off[ks] + fb * 32 * (kQkvBK * 2));
    };
#pragma unroll
    for (int m = 0; m < AHEAD; ++m) fa[m] = frag(m);
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      if (m + AHEAD < NM) fa[m + AHEAD] = frag(m + AHEAD);
      __builtin_amdgcn_sched_barrier(0);
      const int ks = m / kQkvNFB, fb = m % kQkvNFB;
      acc[fb] = mfma32x32x16(fa[m], as_bf16x8(h[ks]), acc[fb]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Epilogue of one tile: lane holds row 32 wave + lane % 32 and, in
  // register i of block fb, column 32 fb + acc_row(i, lane) of the tile.
  // A rotated head's block fb (first half) pairs with block fb + P (second
  // half) at frequency index 32 (fb % BPH) + acc_row(i, lane).
  int ep_tile = blockIdx.x;
  auto epilogue = [&]() __attribute__((always_inline)) {
    const int mt = ep_tile / n_nt;
    const int c0 = (ep_tile - mt * n_nt) * kQkvBN;
    const int64_t t = (int64_t)mt * kQkvBM + wave * 32 + (lane & 31);
    const int64_t tl = t < Kt ? t : Kt - 1;  // rows past Kt are not stored
    const int hf = 4 * (lane >> 5);
#pragma unroll
    for (int bi = 0; bi < P; ++bi) {
      // cos / sin of frequencies 32 bi + 8 i4 + hf + c, c = 0..3, shared by
      // every rotated head of the tile
      float cs[16], sn[16];
      const float4* rr = reinterpret_cast<const float4*>(rope + tl * (HD / 2) + 32 * bi + hf);
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const float4 u0 = rr[4 * i4], u1 = rr[4 * i4 + 1];
        cs[4 * i4 + 0] = u0.x; sn[4 * i4 + 0] = u0.y;
        cs[4 * i4 + 1] = u0.z; sn[4 * i4 + 1] = u0.w;
        cs[4 * i4 + 2] = u1.x; sn[4 * i4 + 2] = u1.y;
        cs[4 * i4 + 3] = u1.z; sn[4 * i4 + 3] = u1.w;
      }
#pragma unroll
      for (int hd = 0; hd < kQkvNFB / BPH; ++hd) {
        const int fb = hd * BPH + bi;
        if (c0 + 32 * fb < rot_cols) {  // q and k heads rotate, v heads do not
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float a = acc[fb][i], b = acc[fb + P][i];
            acc[fb][i] = a * cs[i] - b * sn[i];
            acc[fb + P][i] = b * cs[i] + a * sn[i];
          }
        }
      }
    }
    if (t < Kt) {
      uint16_t* orow = out + t * ld_out + c0 + hf;
#pragma unroll
      for (int fb = 0; fb < kQkvNFB; ++fb) {
        if (c0 + 32 * fb < N) {
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            const __bf16 e0 = (__bf16)acc[fb][4 * i4 + 0], e1 = (__bf16)acc[fb][4 * i4 + 1];
            const __bf16 e2 = (__bf16)acc[fb][4 * i4 + 2], e3 = (__bf16)acc[fb][4 * i4 + 3];
            uint2 pk;
            pk.x = (uint32_t)__builtin_bit_cast(uint16_t, e0) | ((uint32_t)__builtin_bit_cast(uint16_t, e1) << 16);
            pk.y = (uint32_t)__builtin_bit_cast(uint16_t, e2) | ((uint32_t)__builtin_bit_cast(uint16_t, e3) << 16);
            *reinterpret_cast<uint2*>(orow + 32 * fb + 8 * i4) = pk;
          }
        }
      }
    }
    ep_tile += gridDim.x;
  };

  // End of a stage's wait: this wave's loads of the stage about to be
  // computed are complete (PER loads per stage, completing in order; the
  // two newer stages stay in flight) and its LDS reads of the previous
  // stage are done; then all waves meet, so the stage's W_qkv copy is whole
  // and the buffer the next loads fill is no longer read.
#define TG_QKV_SYNC() asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"((kQkvAhead - 1) * PER) : "memory")

  uint4 h0[4], h1[4], h2[4], h3[4];
  issue(sw0, h0);
  issue(sw1, h1);
  issue(sw2, h2);
  int kc = 0;
  for (int s = 0; s < n_steps; s += 4) {
    TG_QKV_SYNC();
    issue(sw3, h3);
    compute(sw0, h0);
    TG_QKV_SYNC();
    issue(sw0, h0);
    compute(sw1, h1);
    TG_QKV_SYNC();
    issue(sw1, h1);
    compute(sw2, h2);
    TG_QKV_SYNC();
    issue(sw2, h2);
    compute(sw3, h3);
    kc += 4;
    if (kc == nk) {
      kc = 0;
      epilogue();
#pragma unroll
      for (int fb = 0; fb < kQkvNFB; ++fb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[fb][i] = 0.0f;
    }
  }
#undef TG_QKV_SYNC
  // the loads issued past the last stage must land before the workgroup's
  // LDS is released
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Tail of the bf16 projection: tiles left over after the last full round of
// the main kernel (at most a quarter of the CUs' worth) would run one per CU
// while the rest of the chip idles, so each is cut into 16 sub-tiles of 64
// rows x one rotation pair of 32-column blocks (blocks fb and fb + d/64 of a
// head), one workgroup each.  The 4 waves of a workgroup split D into
// quarters; each streams its quarter of the pair's 64 W_qkv rows and the 64
// rows of x through its own two LDS stages of 64 columns (buffer-to-LDS
// loads, 8 rows per instruction) and reads MFMA fragments from there.  The
// four partial sums meet in LDS and are added in wave order
// (bit-reproducible), then rotated and stored as in the main kernel.  The
// four workgroups that share a pair's W_qkv rows sit on one XCD (workgroup
// ids 8 apart), so those rows are fetched into one L2.
template <int HD>
__global__ __launch_bounds__(256) void qkv_rope_tail_kernel(
    const uint16_t* __restrict__ x, int64_t ld, int64_t Kt, int D,
    const uint16_t* __restrict__ W, int N, int rot_cols, int n_nt, int first_tile, int n_groups,
    const float2* __restrict__ rope, uint16_t* __restrict__ out, int64_t ld_out) {
  constexpr int BPH = HD / 32;
  constexpr int P = BPH / 2;
  constexpr int SB = 128 * 128;  // one wave's stage: 128 rows (2 W blocks, 2 x blocks) x 64 columns
  __shared__ __attribute__((aligned(16))) char st0[4][SB], st1[4][SB];

  // sub-tile s = xcd + 8 (tq + 4 g2): row quarter tq of (tile, pair) group xcd + 8 g2
  const int sidx = blockIdx.x;
  const int tq = (sidx >> 3) & 3;
  const int grp = (sidx & 7) + 8 * (sidx >> 5);
  if (grp >= n_groups) return;
  const int tile = first_tile + grp / 4;
  const int pr = grp % 4;
  const int mt = tile / n_nt;
  const int nt = tile - mt * n_nt;
  const int fb0 = HD == 128 ? (pr >> 1) * 4 + (pr & 1) : 2 * pr;
  const int f0 = nt * kQkvBN + 32 * fb0;  // first column of the pair's first block
  const int f1 = f0 + 32 * P;
  if (f0 >= N) return;  // heads are whole: the pair lies entirely past N
  const int64_t t0 = (int64_t)mt * kQkvBM + 64 * tq;
  if (t0 >= Kt) return;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rows = (int)min((int64_t)64, Kt - t0);
  const int kq = D / 4;            // this wave's columns [kb, kb + kq), a multiple of 16
  const int kb = wave * kq;
  const int nst = (kq + 63) / 64;  // stages of 64 columns; k-steps past kq are skipped

  // DMA j of a stage fills staged rows 8 j .. 8 j + 7: rows 0-31 are W_qkv
  // rows f0 + r, 32-63 rows f1 + r - 32, 64-127 rows t0 + r - 64 of x.
  // Lane l writes position l % 8 of row 8 j + l / 8, which holds logical
  // chunk (l % 8) ^ ((row >> 1) & 7) of the row's 64 columns.
  int voff[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int row = 8 * j + (lane >> 3);
    const int c = (lane & 7) ^ ((row >> 1) & 7);
    if (j < 4) voff[j] = (row * D + c * 8) * 2;
    else if (j < 8) voff[j] = ((32 * P + row - 32) * D + c * 8) * 2;
    else voff[j] = ((row - 64) * (int)ld + c * 8) * 2;
  }
  // W_qkv rows f0 .. f1 + 31 and x rows t0 .. t0 + rows - 1 from column kb
  // on; reads past the ranges (the last wave's partial stage, rows past Kt)
  // give zeros.
  auto issue = [&](char* buf, int st) __attribute__((always_inline)) {
    const int k0 = kb + 64 * st;
    const int wr = __builtin_amdgcn_readfirstlane((32 * P + 32) * D * 2 - k0 * 2);
    const int xr = __builtin_amdgcn_readfirstlane(rows * (int)ld * 2 - k0 * 2);
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc((void*)(W + (int64_t)f0 * D + k0), (short)0, wr, kBufFlags);
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc((void*)(x + t0 * ld + k0), (short)0, xr, kBufFlags);
#pragma unroll
    for (int j = 0; j < 8; ++j) qkv_lds_load16(rw, buf + 1024 * j, voff[j]);
#pragma unroll
    for (int j = 8; j < 16; ++j) qkv_lds_load16(rx, buf + 1024 * j, voff[j]);
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.0f;
  // fragment of staged block q (0, 1: W_qkv; 2, 3: x), k-step ks
  const int r = lane & 31;
  auto compute = [&](const char* buf, int st) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (64 * st + 16 * ks < kq) {
        const int c = 2 * ks + (lane >> 5);
        bf16x8 f[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int row = 32 * q + r;
          f[q] = *reinterpret_cast<const bf16x8*>(buf + row * 128 + ((c ^ ((row >> 1) & 7)) * 16));
        }
        acc[0][0] = mfma32x32x16(f[0], f[2], acc[0][0]);
        acc[0][1] = mfma32x32x16(f[0], f[3], acc[0][1]);
        acc[1][0] = mfma32x32x16(f[1], f[2], acc[1][0]);
        acc[1][1] = mfma32x32x16(f[1], f[3], acc[1][1]);
      }
    }
  };
  char* b0 = st0[wave];
  char* b1 = st1[wave];
  issue(b0, 0);
  if (nst > 1) issue(b1, 1);
  for (int st = 0; st < nst; st += 2) {
    compute(b0, st);
    if (st + 2 < nst) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads of b0 done before it is refilled
      issue(b0, st + 2);
    }
    if (st + 1 < nst) {
      compute(b1, st + 1);
      if (st + 3 < nst) {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        issue(b1, st + 3);
      }
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();  // every wave is done with its stages: st0 now holds the partial sums
  float* red = reinterpret_cast<float*>(&st0[0][0]);  // [3][4][16][64]
  if (wave > 0) {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) red[(((wave - 1) * 4 + 2 * a + b) * 16 + i) * 64 + lane] = acc[a][b][i];
  }
  __syncthreads();
  if (wave > 0) return;
#pragma unroll
  for (int w = 0; w < 3; ++w)
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[a][b][i] += red[((w * 4 + 2 * a + b) * 16 + i) * 64 + lane];

  const int hf = 4 * (lane >> 5);
  const bool rot = f0 < rot_cols;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int64_t t = t0 + 32 * b + r;
    if (rot) {
      const int64_t tl = t < Kt ? t : Kt - 1;
      const float4* rr = reinterpret_cast<const float4*>(rope + tl * (HD / 2) + 32 * (fb0 % BPH) + hf);
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const float4 u0 = rr[4 * i4], u1 = rr[4 * i4 + 1];
        const float cs[4] = {u0.x, u0.z, u1.x, u1.z}, sn[4] = {u0.y, u0.w, u1.y, u1.w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float av = acc[0][b][4 * i4 + c], bv = acc[1][b][4 * i4 + c];
          acc[0][b][4 * i4 + c] = av * cs[c] - bv * sn[c];
          acc[1][b][4 * i4 + c] = bv * cs[c] + av * sn[c];
        }
      }
    }
    if (t < Kt) {
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        uint16_t* orow = out + t * ld_out + (a ? f1 : f0) + hf;
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const __bf16 e0 = (__bf16)acc[a][b][4 * i4 + 0], e1 = (__bf16)acc[a][b][4 * i4 + 1];
          const __bf16 e2 = (__bf16)acc[a][b][4 * i4 + 2], e3 = (__bf16)acc[a][b][4 * i4 + 3];
          uint2 pk;
          pk.x = (uint32_t)__builtin_bit_cast(uint16_t, e0) | ((uint32_t)__builtin_bit_cast(uint16_t, e1) << 16);
          pk.y = (uint32_t)__builtin_bit_cast(uint16_t, e2) | ((uint32_t)__builtin_bit_cast(uint16_t, e3) << 16);
          *reinterpret_cast<uint2*>(orow + 8 * i4) = pk;
        }
      }
    }
  }
}

// fp32 path: one thread per output element; the dot products over D run
// sequentially in fp32, a rotated element also forms its partner's.
__global__ __launch_bounds__(256) void qkv_rope_f32_kernel(
    const float* __restrict__ x, int64_t ld, int64_t Kt, int D, const float* __restrict__ W,
    int N, int rot_cols, int d, const float2* __restrict__ rope, float* __restrict__ out,
    int64_t ld_out) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= Kt * N) return;
  const int64_t t = idx / N;
  const int n = (int)(idx - t * N);
  const float* xr = x + t * ld;
  auto dot = [&](int row) {
    const float* w = W + (int64_t)row * D;
    float a = 0.0f;
    for (int k = 0; k < D; ++k) a = fmaf(w[k], xr[k], a);
    return a;
  };
  const float y = dot(n);
  if (n >= rot_cols) {
    out[t * ld_out + n] = y;
    return;
  }
  const int half = d / 2;
  const int e = n % d;
  const int i = e < half ? e : e - half;
  const float2 r = rope[t * half + i];
  if (e < half) {
    const float b = dot(n + half);
    out[t * ld_out + n] = y * r.x - b * r.y;
  } else {
    const float a = dot(n - half);
    out[t * ld_out + n] = y * r.x + a * r.y;
  }
}

}  // namespace

hipError_t launch_rope_table(const int32_t* pos, int64_t n, int d, double theta, float* table,
                             hipStream_t s) {
  const int64_t total = n * (d / 2);
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, pos,
                     n, d, theta, reinterpret_cast<float2*>(table));
  return hipGetLastError();
}

hipError_t launch_qkv_rope_bf16(const void* x, int64_t ld, int64_t Kt, int D, const void* W,
                                const float* rope, int Hq, int Hkv, int d, void* out,
                                int64_t ld_out, hipStream_t s) {
  if (Kt == 0) return hipSuccess;
  int n_cu = 0;
  const hipError_t e = device_cu_count(&n_cu);
  if (e != hipSuccess) return e;
  const int N = (Hq + 2 * Hkv) * d;
  const int rot_cols = (Hq + Hkv) * d;
  const int n_mt = (int)((Kt + kQkvBM - 1) / kQkvBM);
  const int n_nt = (N + kQkvBN - 1) / kQkvBN;
  const int n_tiles = n_mt * n_nt;
  if (d != 128 && d != 64) return hipErrorInvalidValue;
  // Tiles past the last full round of one tile per CU go to the sub-tile
  // kernel when there are few of them (at most a quarter of the CUs).
  const int left = n_tiles % n_cu;
  const int main_tiles = (left > 0 && left <= n_cu / 4) ? n_tiles - left : n_tiles;
  const auto* xp = static_cast<const uint16_t*>(x);
  const auto* wp = static_cast<const uint16_t*>(W);
  const auto* rp = reinterpret_cast<const float2*>(rope);
  auto* op = static_cast<uint16_t*>(out);
  if (main_tiles > 0) {
    const dim3 grid((unsigned)min(main_tiles, n_cu));
    if (d == 128)
      hipLaunchKernelGGL((qkv_rope_bf16_kernel<128>), grid, dim3(512), 0, s, xp, ld, Kt, D, wp, N,
                         rot_cols, n_nt, main_tiles, rp, op, ld_out);
    else
      hipLaunchKernelGGL((qkv_rope_bf16_kernel<64>), grid, dim3(512), 0, s, xp, ld, Kt, D, wp, N,
                         rot_cols, n_nt, main_tiles, rp, op, ld_out);
    const hipError_t e1 = hipGetLastError();
    if (e1 != hipSuccess) return e1;
  }
  if (main_tiles < n_tiles) {
    // 4 (tile, pair) groups per tile, 4 row quarters each; ids are laid out
    // in blocks of 32 (8 groups x 4 quarters), the last block padded
    const int n_groups = (n_tiles - main_tiles) * 4;
    const dim3 grid((unsigned)((n_groups + 7) / 8 * 32));
    if (d == 128)
      hipLaunchKernelGGL((qkv_rope_tail_kernel<128>), grid, dim3(256), 0, s, xp, ld, Kt, D, wp, N,
                         rot_cols, n_nt, main_tiles, n_groups, rp, op, ld_out);
    else
      hipLaunchKernelGGL((qkv_rope_tail_kernel<64>), grid, dim3(256), 0, s, xp, ld, Kt, D, wp, N,
                         rot_cols, n_nt, main_tiles, n_groups, rp, op, ld_out);
  }
  return hipGetLastError();
}

hipError_t launch_qkv_rope_f32(const float* x, int64_t ld, int64_t Kt, int D, const float* W,
                               const float* rope, int Hq, int Hkv, int d, float* out,
                               int64_t ld_out, hipStream_t s) {
  const int N = (Hq + 2 * Hkv) * d;
  const int64_t total = Kt * N;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(qkv_rope_f32_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                     x, ld, Kt, D, W, N, (Hq + Hkv) * d, d, reinterpret_cast<const float2*>(rope),
                     out, ld_out);
  return hipGetLastError();
}

}  // namespace tg
