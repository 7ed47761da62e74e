// The pruned layers above the gate, on the kept rows (TokenGate article,
// section "How does TokenGate learned token pruning work?": those layers run
// on the kept tokens only, each at the position id it had in the full
// prompt).  A pre-norm layer of the Qwen3 family:
//     a = x + W_o . attention(rope(W_qkv . rms_norm(x)))
//     y = a + W_down . (silu(W_gate . rms_norm(a)) * (W_up . rms_norm(a)))
// Every product is a projection of the kept rows, C^T[n][t] = W[n] . x[t];
// they share one main loop and differ in the epilogue:
//   rope    (q/k/v) the q and k heads are rotated in the rotate-half form
//           (element i of a head pairs with i + d/2, angle
//           pos * theta^(-2 i / d), cos / sin from a per-row table), v stored
//           as projected;
//   resid   (attention output and down projection) the residual row is added;
//   swiglu  (gate and up projections) silu(gate) * up;
//   store   plain product (the gate backward's dh = da . W1).
//
// Kernels:
//   rope_table   cos / sin of every (kept row, frequency) pair, evaluated in
//                fp64 from the row's position and stored as fp32 pairs
//                [Kt, d/2]; it depends on the positions only, so a pruned
//                forward builds it once for all its layers.
//   rms_norm     one wave per row: fp32 sum of squares in a fixed reduction
//                order, then w * x / sqrt(mean + eps) rounded once.
//   proj_bf16    the 32x32x16 bf16 MFMA, the gate MLP's pipeline: rows of x
//                straight from memory into the registers that serve as the B
//                operand, three 64-column stages ahead; weight rows through
//                four LDS stages filled by buffer-to-LDS loads.  A workgroup
//                of 8 waves owns tiles of 256 rows x 256 weight rows (each wave
//                32 rows of x and all 256 weight rows), one workgroup per CU
//                looping over tiles.  An epilogue combines pairs of 32-column
//                blocks that sit in the same lane and register: a rotation
//                pair (blocks j and j + d/64 of a head: heads never straddle
//                a tile since d divides 256) or a gate / up pair (the tile
//                stages 128 rows of W_gate and the same 128 rows of W_up).
//   proj_tail    tiles past the last full round of one tile per CU, cut into
//                sub-tiles so that they spread over the chip.
//   fp32 paths   one thread per output element on vector ALUs.

#include "tg_common.h"

namespace tg {
namespace {

constexpr int kBK = 64;     // reduction columns per stage (128-byte row segments)
constexpr int kAhead = 3;   // stages loaded ahead of the one computed
constexpr int kBM = 256;    // rows of x per tile (8 waves x 32)
constexpr int kNFB = 8;     // 32-row weight blocks per tile
constexpr int kBufFlags = 0x00020000;  // raw buffer: reads past num_records give 0

enum ProjEpi : int { kEpiRope = 0, kEpiResid = 1, kEpiSwiglu = 2, kEpiStore = 3 };

// Weight rows staged per source in a tile: 256 of W, or 128 of W_gate
// followed by the same 128 of W_up.
template <int EPI>
constexpr int rows_per_src() { return EPI == kEpiSwiglu ? 128 : 256; }

struct ProjArgs {
  const uint16_t* x;     // rows of the kept tokens, [M, K], row stride ld
  int64_t ld;
  int64_t M;
  int K;
  const uint16_t* w0;    // weight rows [nw, K] (W_gate for swiglu)
  const uint16_t* w1;    // W_up for swiglu, else unused
  int nw;
  int N;                 // output columns
  int n_nt;              // column tiles
  int n_tiles;           // tiles of the tile kernel / first tile of the tail
  int n_groups;          // tail: (tile, pair) groups
  const float2* rope;    // rope: [M, d/2] (cos, sin)
  int rot_cols;          // rope: columns below rot_cols are rotated (q and k heads)
  const uint16_t* res;   // resid: residual rows, stride ld_res
  int64_t ld_res;
  uint16_t* out;         // output rows, stride ld_out
  int64_t ld_out;
};

// A staged row of weights is 64 columns = eight 16-byte chunks; logical
// chunk c of row r sits at position c ^ ((r >> 1) & 7), so that the fragment
// reads of 16 consecutive rows at one chunk touch 16 different bank groups.
__device__ __forceinline__ int proj_swz(int r, int c) { return c ^ ((r >> 1) & 7); }

// One 16-byte buffer-to-LDS load per lane: lane l writes bytes
// [16 l, 16 l + 16) of lds.  Out-of-range reads write zeros.
__device__ __forceinline__ void proj_lds_load16(__amdgpu_buffer_rsrc_t r, char* lds, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, 0, 0, 0);
}

// LDS byte offset of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_off(const char* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)p;
}

// Four 16-byte LDS reads and the wait for them, in one asm block (so the
// compiler neither reorders nor re-waits them).
__device__ __forceinline__ void lds_read4_wait(const uint32_t (&a)[4], bf16x8 (&f)[4]) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  u32x4 r0, r1, r2, r3;
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %5\n\t"
      "ds_read_b128 %2, %6\n\t"
      "ds_read_b128 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
      : "memory");
  f[0] = __builtin_bit_cast(bf16x8, r0);
  f[1] = __builtin_bit_cast(bf16x8, r1);
  f[2] = __builtin_bit_cast(bf16x8, r2);
  f[3] = __builtin_bit_cast(bf16x8, r3);
}

__device__ __forceinline__ uint2 pack_bf16x4(float a, float b, float c, float d) {
  const __bf16 e0 = (__bf16)a, e1 = (__bf16)b, e2 = (__bf16)c, e3 = (__bf16)d;
  uint2 pk;
  pk.x = (uint32_t)__builtin_bit_cast(uint16_t, e0) | ((uint32_t)__builtin_bit_cast(uint16_t, e1) << 16);
  pk.y = (uint32_t)__builtin_bit_cast(uint16_t, e2) | ((uint32_t)__builtin_bit_cast(uint16_t, e3) << 16);
  return pk;
}

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

__device__ __forceinline__ float silu(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// The two 32-column blocks (of a 256-row weight tile) that the epilogue
// combines: pair p = 0..3.
template <int EPI, int HD>
__device__ __forceinline__ int pair_first(int p) {
  if (EPI == kEpiRope && HD == 128) return (p >> 1) * 4 + (p & 1);  // blocks j, j + 2 of a head
  if (EPI == kEpiSwiglu) return p;                                  // gate block p, up block p + 4
  return 2 * p;                                                     // adjacent blocks
}
template <int EPI, int HD>
constexpr int pair_dist() { return EPI == kEpiSwiglu ? 4 : (EPI == kEpiRope && HD == 128 ? 2 : 1); }

// Epilogue of one pair of blocks for one 32-row block of x: a and b hold, in
// register i of lane l, rows acc_row(i, l) of blocks A and B at row
// t = (token of lane l).  colA / colB: output columns of the blocks' first
// rows (colB unused for swiglu); freq0: rope frequency index of block A's
// first row.
template <int EPI, int HD>
__device__ __forceinline__ void finish_pair(const ProjArgs& g, f32x16& a, f32x16& b, int64_t t,
                                            int colA, int colB, int freq0, int lane) {
  const int hf = 4 * (lane >> 5);
  if (EPI == kEpiRope) {
    if (colA < g.rot_cols) {
      const int64_t tl = t < g.M ? t : g.M - 1;
      const float4* rr = reinterpret_cast<const float4*>(g.rope + tl * (HD / 2) + freq0 + hf);
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const float4 u0 = rr[4 * i4], u1 = rr[4 * i4 + 1];
        const float cs[4] = {u0.x, u0.z, u1.x, u1.z}, sn[4] = {u0.y, u0.w, u1.y, u1.w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float av = a[4 * i4 + c], bv = b[4 * i4 + c];
          a[4 * i4 + c] = av * cs[c] - bv * sn[c];
          b[4 * i4 + c] = bv * cs[c] + av * sn[c];
        }
      }
    }
  }
  // rows past M store nothing (the lanes of a row pair share t)
  const bool ok = t < g.M;
  const int64_t tr = ok ? t : 0;
  const int G = lane >> 5;
  if (EPI == kEpiSwiglu) {
    store_row32_bf16(g.out + tr * g.ld_out + colA, G, ok,
                     [&](int i) __attribute__((always_inline)) { return silu(a[i]) * b[i]; });
    return;
  }
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    f32x16& v = s ? b : a;
    const int col = s ? colB : colA;
    if (EPI == kEpiResid && ok) {
      const uint16_t* rrow = g.res + t * g.ld_res + col + hf;
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const uint2 r = *reinterpret_cast<const uint2*>(rrow + 8 * i4);
        v[4 * i4] += bf16_lo(r.x);
        v[4 * i4 + 1] += bf16_hi(r.x);
        v[4 * i4 + 2] += bf16_lo(r.y);
        v[4 * i4 + 3] += bf16_hi(r.y);
      }
    }
    store_row32_bf16(g.out + tr * g.ld_out + col, G, ok, [&](int i) __attribute__((always_inline)) { return v[i]; });
  }
}

// Output column of a weight tile's 32-row block fb (its first row), and
// whether the block exists (weight rows past nw are zeros and not stored).
template <int EPI>
__device__ __forceinline__ int block_col(int nt, int fb) {
  return EPI == kEpiSwiglu ? nt * 128 + 32 * (fb & 3) : nt * 256 + 32 * fb;
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

// RMSNorm, one wave per row.  Lane l owns the 8-element chunks l, l + 64,
// ... of the row; the fp32 sum of squares is reduced over the lanes by a
// fixed butterfly, so every row sees the same order.
template <typename T>
__global__ __launch_bounds__(256) void rms_norm_kernel(const T* __restrict__ x, int64_t ld, int64_t n,
                                                       int D, const float* __restrict__ w, float eps,
                                                       T* __restrict__ out, int64_t ld_out) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= n) return;
  const T* xr = x + row * ld;
  T* orow = out + row * ld_out;
  float ss = 0.0f;
  for (int e = 8 * lane; e < D; e += 512) {
    float v[8];
    if constexpr (sizeof(T) == 2) {
      const uint4 u = *reinterpret_cast<const uint4*>(xr + e);
      const uint32_t q[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[2 * j] = bf16_lo(q[j]);
        v[2 * j + 1] = bf16_hi(q[j]);
      }
    } else {
      const float4 a = *reinterpret_cast<const float4*>(xr + e);
      const float4 b = *reinterpret_cast<const float4*>(xr + e + 4);
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
      v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) ss = fmaf(v[j], v[j], ss);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
  const float inv = 1.0f / sqrtf(ss / (float)D + eps);
  for (int e = 8 * lane; e < D; e += 512) {
    const float4 w0 = *reinterpret_cast<const float4*>(w + e);
    const float4 w1 = *reinterpret_cast<const float4*>(w + e + 4);
    const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
    if constexpr (sizeof(T) == 2) {
      const uint4 u = *reinterpret_cast<const uint4*>(xr + e);
      const uint32_t q[4] = {u.x, u.y, u.z, u.w};
      float v[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[2 * j] = bf16_lo(q[j]) * inv * wv[2 * j];
        v[2 * j + 1] = bf16_hi(q[j]) * inv * wv[2 * j + 1];
      }
      const uint2 lo = pack_bf16x4(v[0], v[1], v[2], v[3]);
      const uint2 hi = pack_bf16x4(v[4], v[5], v[6], v[7]);
      *reinterpret_cast<uint4*>(orow + e) = make_uint4(lo.x, lo.y, hi.x, hi.y);
    } else {
      const float4 a = *reinterpret_cast<const float4*>(xr + e);
      const float4 b = *reinterpret_cast<const float4*>(xr + e + 4);
      *reinterpret_cast<float4*>(orow + e) =
          make_float4(a.x * inv * wv[0], a.y * inv * wv[1], a.z * inv * wv[2], a.w * inv * wv[3]);
      *reinterpret_cast<float4*>(orow + e + 4) =
          make_float4(b.x * inv * wv[4], b.y * inv * wv[5], b.z * inv * wv[6], b.w * inv * wv[7]);
    }
  }
}

// Reduction order inside a stage: a lane of half h = lane / 32 supplies, for
// k-step j, the 8 columns [32 h + 8 j, 32 h + 8 j + 8) of its stage, for x
// and for the weight fragments alike, so the products sum over the columns
// of the definition, in another order.
template <int EPI, int HD>
__global__ __launch_bounds__(512, 1) void proj_bf16_kernel(ProjArgs g) {
  constexpr int NW = 8;
  constexpr int W_BYTES = 256 * kBK * 2;     // one stage of weight rows
  constexpr int W_DMA = W_BYTES / 1024 / NW;  // 1 KB buffer-to-LDS copies per wave per stage
  constexpr int PER = W_DMA + 4;              // vector-memory instructions per wave per stage
  constexpr int RPS = rows_per_src<EPI>();
  static_assert(W_DMA * 8 == 32, "a wave stages 32 weight rows");

  __shared__ __attribute__((aligned(16))) char sw0[W_BYTES], sw1[W_BYTES], sw2[W_BYTES], sw3[W_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int K = g.K;
  const int n_tiles = g.n_tiles;
  const int n_nt = g.n_nt;

  // Stages per tile, rounded up to a multiple of four (the unroll below);
  // stages past K load zeros and add nothing.
  const int nk = (K / kBK + 3) & ~3;
  const int my_tiles = ((int)blockIdx.x < n_tiles) ? (n_tiles - 1 - (int)blockIdx.x) / (int)gridDim.x + 1 : 0;
  const int n_steps = my_tiles * nk;

  // x: lane loads 64 contiguous bytes of row 32 wave + lane % 32 of the tile
  const int h_voff = ((wave * 32 + (lane & 31)) * (int)g.ld + (lane >> 5) * 32) * 2;
  // Weight copies: this wave stages rows 32 wave .. 32 wave + 31 of the
  // tile, from W (or, for swiglu, waves 0-3 from W_gate and 4-7 from W_up);
  // copy j fills rows 32 wave + 8 j .. +7, lane l position l % 8 of row
  // l / 8, which holds that row's logical chunk proj_swz(row, l % 8).
  const uint16_t* wsrc = (EPI == kEpiSwiglu && wave >= 4) ? g.w1 : g.w0;
  int w_src[W_DMA];
#pragma unroll
  for (int j = 0; j < W_DMA; ++j) {
    const int r = (wave * W_DMA + j) * 8 + (lane >> 3);
    w_src[j] = ((r % RPS) * K + proj_swz(r, lane & 7) * 8) * 2;
  }
  // weight fragment of block fb, k-step ks: row 32 fb + lane % 32, logical
  // chunk 4 (lane / 32) + ks; the swizzle term depends on the lane only
  int a_off[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    a_off[ks] = (lane & 31) * (kBK * 2) + proj_swz(lane & 31, 4 * (lane >> 5) + ks) * 16;

  // Load position: tile ld_tile (a multiple of gridDim.x past blockIdx.x),
  // stage ld_k of it; tile id = row tile * n_nt + column tile.  Loads past
  // the last tile read nothing (zero range).
  int ld_tile = blockIdx.x, ld_k = 0;
  int ld_mt = ld_tile / n_nt, ld_nt = ld_tile - ld_mt * n_nt;
  auto issue = [&](char* sw, uint4 (&h)[4]) __attribute__((always_inline)) {
    const bool tin = ld_tile < n_tiles;
    const int64_t t0 = (int64_t)ld_mt * kBM;
    const int r0 = ld_nt * RPS;  // first weight row of the tile in each source
    const int rows = tin ? (int)min((int64_t)kBM, g.M - t0) : 0;
    const int wrows = tin ? min(RPS, g.nw - r0) : 0;
    const int k0 = ld_k * kBK;
    const bool kin = k0 < K;
    const int kk = kin ? k0 : 0;
    const int hb = __builtin_amdgcn_readfirstlane((rows > 0 && kin) ? rows * (int)g.ld * 2 - kk * 2 : 0);
    const int wb = __builtin_amdgcn_readfirstlane((wrows > 0 && kin) ? wrows * K * 2 - kk * 2 : 0);
    const uint16_t* hb_ptr = rows > 0 ? g.x + t0 * g.ld + kk : g.x;
    const uint16_t* wb_ptr = wrows > 0 ? wsrc + (int64_t)r0 * K + kk : wsrc;
    const __amdgpu_buffer_rsrc_t rh = __builtin_amdgcn_make_buffer_rsrc((void*)hb_ptr, (short)0, hb, kBufFlags);
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc((void*)wb_ptr, (short)0, wb, kBufFlags);
#pragma unroll
    for (int j = 0; j < W_DMA; ++j)
      proj_lds_load16(rw, sw + (wave * W_DMA + j) * 1024, w_src[j]);
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

  f32x16 acc[kNFB];
#pragma unroll
  for (int fb = 0; fb < kNFB; ++fb)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[fb][i] = 0.0f;

  // One stage: 4 k-steps x 8 weight blocks; each weight fragment is read
  // three MFMAs ahead of its use.
  constexpr int NM = 4 * kNFB;
  constexpr int AHEAD = 3;
  auto compute = [&](const char* sw, const uint4 (&h)[4]) __attribute__((always_inline)) {
    bf16x8 fa[NM];
    auto frag = [&](int m) __attribute__((always_inline)) {
      const int ks = m / kNFB, fb = m % kNFB;
      return *reinterpret_cast<const bf16x8*>(sw + a_off[ks] + fb * 32 * (kBK * 2));
    };
#pragma unroll
    for (int m = 0; m < AHEAD; ++m) fa[m] = frag(m);
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      if (m + AHEAD < NM) fa[m + AHEAD] = frag(m + AHEAD);
      __builtin_amdgcn_sched_barrier(0);
      const int ks = m / kNFB, fb = m % kNFB;
      acc[fb] = mfma32x32x16(fa[m], as_bf16x8(h[ks]), acc[fb]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Epilogue of one tile: lane holds row 32 wave + lane % 32 and, in
  // register i of block fb, weight row 32 fb + acc_row(i, lane) of the tile.
  int ep_tile = blockIdx.x;
  auto epilogue = [&]() __attribute__((always_inline)) {
    const int mt = ep_tile / n_nt;
    const int nt = ep_tile - mt * n_nt;
    const int64_t t = (int64_t)mt * kBM + wave * 32 + (lane & 31);
    constexpr int PD = pair_dist<EPI, HD>();
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int fa_ = pair_first<EPI, HD>(p);
      const int colA = block_col<EPI>(nt, fa_);
      if (colA < g.N)  // pairs are whole: both blocks exist or neither
        finish_pair<EPI, HD>(g, acc[fa_], acc[fa_ + PD], t, colA, block_col<EPI>(nt, fa_ + PD),
                             32 * (fa_ % (HD / 32)), lane);
    }
    ep_tile += gridDim.x;
  };

  // End of a stage's wait: this wave's loads of the stage about to be
  // computed are complete (PER loads per stage, completing in order; the
  // two newer stages stay in flight) and its LDS reads of the previous
  // stage are done; then all waves meet, so the stage's weight copy is
  // whole and the buffer the next loads fill is no longer read.
#define TG_PROJ_SYNC() asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"((kAhead - 1) * PER) : "memory")

  uint4 h0[4], h1[4], h2[4], h3[4];
  issue(sw0, h0);
  issue(sw1, h1);
  issue(sw2, h2);
  int kc = 0;
  for (int s = 0; s < n_steps; s += 4) {
    TG_PROJ_SYNC();
    issue(sw3, h3);
    compute(sw0, h0);
    TG_PROJ_SYNC();
    issue(sw0, h0);
    compute(sw1, h1);
    TG_PROJ_SYNC();
    issue(sw1, h1);
    compute(sw2, h2);
    TG_PROJ_SYNC();
    issue(sw2, h2);
    compute(sw3, h3);
    kc += 4;
    if (kc == nk) {
      kc = 0;
      epilogue();
#pragma unroll
      for (int fb = 0; fb < kNFB; ++fb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[fb][i] = 0.0f;
    }
  }
#undef TG_PROJ_SYNC
  // the loads issued past the last stage must land before the workgroup's
  // LDS is released
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Tail: tiles past the last full round of one tile per CU (at most a
// quarter of the CUs' worth) would run one per CU while the rest of the chip
// idles, so each is cut into 16 sub-tiles of 64 rows x one pair of 32-row
// weight blocks, one workgroup each.  The 4 waves of a workgroup split K
// into quarters; each streams its quarter of the pair's 64 weight rows and
// the 64 rows of x through its own two LDS stages of 64 columns
// (buffer-to-LDS loads, 8 rows per instruction) and reads MFMA fragments
// from there.  The four partial sums meet in LDS and are added in wave order
// (bit-reproducible), then finished as in the tile kernel.  The four
// workgroups that share a pair's weight rows sit on one XCD (workgroup ids 8
// apart), so those rows are fetched into one L2.
template <int EPI, int HD>
__global__ __launch_bounds__(256) void proj_tail_kernel(ProjArgs g) {
  constexpr int RPS = rows_per_src<EPI>();
  constexpr int PD = pair_dist<EPI, HD>();
  constexpr int SB = 128 * 128;  // one wave's stage: 128 rows (2 weight blocks, 2 x blocks) x 64 columns
  __shared__ __attribute__((aligned(16))) char st0[4][SB], st1[4][SB];

  // sub-tile s = xcd + 8 (tq + 4 g2): row quarter tq of (tile, pair) group xcd + 8 g2
  const int sidx = blockIdx.x;
  const int tq = (sidx >> 3) & 3;
  const int grp = (sidx & 7) + 8 * (sidx >> 5);
  if (grp >= g.n_groups) return;
  const int tile = g.n_tiles + grp / 4;
  const int pr = grp % 4;
  const int mt = tile / g.n_nt;
  const int nt = tile - mt * g.n_nt;
  const int fbA = pair_first<EPI, HD>(pr);
  const int fbB = fbA + PD;
  const int colA = block_col<EPI>(nt, fbA);
  if (colA >= g.N) return;  // pairs are whole: the pair lies entirely past N
  const int64_t t0 = (int64_t)mt * kBM + 64 * tq;
  if (t0 >= g.M) return;
  // first weight row of each block in its source
  const int rA = nt * RPS + 32 * (fbA % (RPS / 32));
  const int rB = nt * RPS + 32 * (fbB % (RPS / 32));
  const uint16_t* srcB = (EPI == kEpiSwiglu) ? g.w1 : g.w0;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int K = g.K;
  const int rows = (int)min((int64_t)64, g.M - t0);
  const int kq = K / 4;            // this wave's columns [kb, kb + kq), a multiple of 16
  const int kb = wave * kq;
  const int nst = (kq + 63) / 64;  // stages of 64 columns; k-steps past kq are skipped

  // DMA j of a stage fills staged rows 8 j .. 8 j + 7: rows 0-31 are weight
  // rows rA + r, 32-63 rows rB + r - 32, 64-127 rows t0 + r - 64 of x.
  // Lane l writes position l % 8 of row 8 j + l / 8, which holds logical
  // chunk (l % 8) ^ ((row >> 1) & 7) of the row's 64 columns.
  int voff[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int row = 8 * j + (lane >> 3);
    const int c = proj_swz(row, lane & 7);
    if (j < 8) voff[j] = ((row & 31) * K + c * 8) * 2;
    else voff[j] = ((row - 64) * (int)g.ld + c * 8) * 2;
  }
  // Reads past the ranges (the last wave's partial stage, rows past M) give
  // zeros; in-range columns past kq are read but not used.
  auto issue = [&](char* buf, int st) __attribute__((always_inline)) {
    const int k0 = kb + 64 * st;
    const int wr = __builtin_amdgcn_readfirstlane(32 * K * 2 - k0 * 2);
    const int xr = __builtin_amdgcn_readfirstlane(rows * (int)g.ld * 2 - k0 * 2);
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc((void*)(g.w0 + (int64_t)rA * K + k0), (short)0, wr, kBufFlags);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc((void*)(srcB + (int64_t)rB * K + k0), (short)0, wr, kBufFlags);
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc((void*)(g.x + t0 * g.ld + k0), (short)0, xr, kBufFlags);
#pragma unroll
    for (int j = 0; j < 4; ++j) proj_lds_load16(ra, buf + 1024 * j, voff[j]);
#pragma unroll
    for (int j = 4; j < 8; ++j) proj_lds_load16(rb, buf + 1024 * j, voff[j]);
#pragma unroll
    for (int j = 8; j < 16; ++j) proj_lds_load16(rx, buf + 1024 * j, voff[j]);
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.0f;
  // fragment of staged block q (0, 1: weights A, B; 2, 3: x), k-step ks
  const int r = lane & 31;
  auto compute = [&](const char* buf, int st) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (64 * st + 16 * ks < kq) {
        const int c = 2 * ks + (lane >> 5);
        uint32_t ad[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int row = 32 * q + r;
          ad[q] = lds_off(buf + row * 128 + proj_swz(row, c) * 16);
        }
        bf16x8 f[4];
        lds_read4_wait(ad, f);
        acc[0][0] = mfma32x32x16(f[0], f[2], acc[0][0]);
        acc[0][1] = mfma32x32x16(f[0], f[3], acc[0][1]);
        acc[1][0] = mfma32x32x16(f[1], f[2], acc[1][0]);
        acc[1][1] = mfma32x32x16(f[1], f[3], acc[1][1]);
      }
    }
  };
  char* b0 = st0[wave];
  char* b1 = st1[wave];
  // The fragment reads are inline asm that waits for its own LDS reads, so
  // the compiler adds no wait for the buffer-to-LDS loads: the waits below
  // are explicit and counted (16 loads per stage, issued in order), so a
  // stage's loads stay in flight while the other stage is computed.
  issue(b0, 0);
  if (nst > 1) issue(b1, 1);
  for (int st = 0; st < nst; st += 2) {
    if (st + 1 < nst) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    compute(b0, st);
    if (st + 2 < nst) issue(b0, st + 2);  // compute's reads have completed
    if (st + 1 < nst) {
      if (st + 2 < nst) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      compute(b1, st + 1);
      if (st + 3 < nst) issue(b1, st + 3);
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
#pragma unroll
  for (int b = 0; b < 2; ++b)
    finish_pair<EPI, HD>(g, acc[0][b], acc[1][b], t0 + 32 * b + r, colA, block_col<EPI>(nt, fbB),
                         32 * (fbA % (HD / 32)), lane);
}

// fp32 paths: one thread per output element; dot products over K run
// sequentially in fp32.
__device__ __forceinline__ float dot_f32(const float* w, const float* xr, int K) {
  float a = 0.0f;
  for (int k = 0; k < K; ++k) a = fmaf(w[k], xr[k], a);
  return a;
}

__global__ __launch_bounds__(256) void qkv_rope_f32_kernel(
    const float* __restrict__ x, int64_t ld, int64_t M, int K, const float* __restrict__ W,
    int N, int rot_cols, int d, const float2* __restrict__ rope, float* __restrict__ out,
    int64_t ld_out) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= M * N) return;
  const int64_t t = idx / N;
  const int n = (int)(idx - t * N);
  const float* xr = x + t * ld;
  const float y = dot_f32(W + (int64_t)n * K, xr, K);
  if (n >= rot_cols) {
    out[t * ld_out + n] = y;
    return;
  }
  const int half = d / 2;
  const int e = n % d;
  const int i = e < half ? e : e - half;
  const float2 r = rope[t * half + i];
  if (e < half) {
    const float b = dot_f32(W + (int64_t)(n + half) * K, xr, K);
    out[t * ld_out + n] = y * r.x - b * r.y;
  } else {
    const float a = dot_f32(W + (int64_t)(n - half) * K, xr, K);
    out[t * ld_out + n] = y * r.x + a * r.y;
  }
}

__global__ __launch_bounds__(256) void linear_residual_f32_kernel(
    const float* __restrict__ a, int64_t ld, int64_t M, int K, const float* __restrict__ W, int N,
    const float* res, int64_t ld_res, float* out, int64_t ld_out) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= M * N) return;
  const int64_t t = idx / N;
  const int n = (int)(idx - t * N);
  const float y = dot_f32(W + (int64_t)n * K, a + t * ld, K);
  out[t * ld_out + n] = res[t * ld_res + n] + y;
}

__global__ __launch_bounds__(256) void swiglu_f32_kernel(
    const float* __restrict__ h, int64_t ld, int64_t M, int K, const float* __restrict__ Wg,
    const float* __restrict__ Wu, int N, float* __restrict__ out, int64_t ld_out) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= M * N) return;
  const int64_t t = idx / N;
  const int n = (int)(idx - t * N);
  const float gv = dot_f32(Wg + (int64_t)n * K, h + t * ld, K);
  const float uv = dot_f32(Wu + (int64_t)n * K, h + t * ld, K);
  out[t * ld_out + n] = gv / (1.0f + expf(-gv)) * uv;
}

// Launch the bf16 projection: the tile kernel over whole rounds, the tail
// kernel over the tiles left past the last full round when they fill at
// most a quarter of the CUs.
template <int EPI, int HD>
hipError_t launch_proj(ProjArgs g, hipStream_t s) {
  if (g.M == 0) return hipSuccess;
  int n_cu = 0;
  const hipError_t e = device_cu_count(&n_cu);
  if (e != hipSuccess) return e;
  constexpr int RPS = rows_per_src<EPI>();
  const int n_mt = (int)((g.M + kBM - 1) / kBM);
  g.n_nt = (g.nw + RPS - 1) / RPS;
  const int n_tiles = n_mt * g.n_nt;
  const int left = n_tiles % n_cu;
  const int main_tiles = (left > 0 && left <= n_cu / 4) ? n_tiles - left : n_tiles;
  if (main_tiles > 0) {
    g.n_tiles = main_tiles;
    g.n_groups = 0;
    hipLaunchKernelGGL((proj_bf16_kernel<EPI, HD>), dim3((unsigned)min(main_tiles, n_cu)), dim3(512), 0, s, g);
    const hipError_t e1 = hipGetLastError();
    if (e1 != hipSuccess) return e1;
  }
  if (main_tiles < n_tiles) {
    // 4 (tile, pair) groups per tile, 4 row quarters each; ids are laid out
    // in blocks of 32 (8 groups x 4 quarters), the last block padded
    g.n_tiles = main_tiles;
    g.n_groups = (n_tiles - main_tiles) * 4;
    hipLaunchKernelGGL((proj_tail_kernel<EPI, HD>), dim3((unsigned)((g.n_groups + 7) / 8 * 32)), dim3(256), 0, s, g);
  }
  return hipGetLastError();
}

ProjArgs proj_args(const void* x, int64_t ld, int64_t M, int K, const void* w0, const void* w1,
                   int nw, void* out, int64_t ld_out) {
  ProjArgs g{};
  g.x = static_cast<const uint16_t*>(x);
  g.ld = ld;
  g.M = M;
  g.K = K;
  g.w0 = static_cast<const uint16_t*>(w0);
  g.w1 = static_cast<const uint16_t*>(w1);
  g.nw = nw;
  g.N = nw;
  g.out = static_cast<uint16_t*>(out);
  g.ld_out = ld_out;
  return g;
}

dim3 elementwise_grid(int64_t total) { return dim3((unsigned)((total + 255) / 256)); }

}  // namespace

hipError_t launch_rope_table(const int32_t* pos, int64_t n, int d, double theta, float* table,
                             hipStream_t s) {
  const int64_t total = n * (d / 2);
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(rope_table_kernel, elementwise_grid(total), dim3(256), 0, s, pos, n, d, theta,
                     reinterpret_cast<float2*>(table));
  return hipGetLastError();
}

hipError_t launch_rms_norm(const void* x, int64_t ld, int64_t n, int D, const float* w, float eps,
                           int elem_bytes, void* out, int64_t ld_out, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)((n + 3) / 4));
  if (elem_bytes == 2)
    hipLaunchKernelGGL(rms_norm_kernel<uint16_t>, grid, dim3(256), 0, s,
                       static_cast<const uint16_t*>(x), ld, n, D, w, eps, static_cast<uint16_t*>(out), ld_out);
  else
    hipLaunchKernelGGL(rms_norm_kernel<float>, grid, dim3(256), 0, s, static_cast<const float*>(x), ld,
                       n, D, w, eps, static_cast<float*>(out), ld_out);
  return hipGetLastError();
}

hipError_t launch_qkv_rope_bf16(const void* x, int64_t ld, int64_t Kt, int D, const void* W,
                                const float* rope, int Hq, int Hkv, int d, void* out,
                                int64_t ld_out, hipStream_t s) {
  ProjArgs g = proj_args(x, ld, Kt, D, W, nullptr, (Hq + 2 * Hkv) * d, out, ld_out);
  g.rope = reinterpret_cast<const float2*>(rope);
  g.rot_cols = (Hq + Hkv) * d;
  if (d == 128) return launch_proj<kEpiRope, 128>(g, s);
  if (d == 64) return launch_proj<kEpiRope, 64>(g, s);
  return hipErrorInvalidValue;
}

hipError_t launch_qkv_rope_f32(const float* x, int64_t ld, int64_t Kt, int D, const float* W,
                               const float* rope, int Hq, int Hkv, int d, float* out,
                               int64_t ld_out, hipStream_t s) {
  const int N = (Hq + 2 * Hkv) * d;
  const int64_t total = Kt * N;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(qkv_rope_f32_kernel, elementwise_grid(total), dim3(256), 0, s, x, ld, Kt, D, W,
                     N, (Hq + Hkv) * d, d, reinterpret_cast<const float2*>(rope), out, ld_out);
  return hipGetLastError();
}

hipError_t launch_linear_residual(const void* a, int64_t ld, int64_t n, int K, const void* W, int N,
                                  const void* res, int64_t ld_res, int elem_bytes, void* out,
                                  int64_t ld_out, hipStream_t s) {
  if (elem_bytes == 2) {
    ProjArgs g = proj_args(a, ld, n, K, W, nullptr, N, out, ld_out);
    g.res = static_cast<const uint16_t*>(res);
    g.ld_res = ld_res;
    return launch_proj<kEpiResid, 128>(g, s);
  }
  const int64_t total = n * N;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(linear_residual_f32_kernel, elementwise_grid(total), dim3(256), 0, s,
                     static_cast<const float*>(a), ld, n, K, static_cast<const float*>(W), N,
                     static_cast<const float*>(res), ld_res, static_cast<float*>(out), ld_out);
  return hipGetLastError();
}

hipError_t launch_proj_store(const void* x, int64_t ld, int64_t n, int K, const void* W, int N, void* out,
                             int64_t ld_out, hipStream_t s) {
  return launch_proj<kEpiStore, 128>(proj_args(x, ld, n, K, W, nullptr, N, out, ld_out), s);
}

hipError_t launch_swiglu(const void* h, int64_t ld, int64_t n, int K, const void* Wg, const void* Wu,
                         int I, int elem_bytes, void* out, int64_t ld_out, hipStream_t s) {
  if (elem_bytes == 2) return launch_proj<kEpiSwiglu, 128>(proj_args(h, ld, n, K, Wg, Wu, I, out, ld_out), s);
  const int64_t total = n * I;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(swiglu_f32_kernel, elementwise_grid(total), dim3(256), 0, s,
                     static_cast<const float*>(h), ld, n, K, static_cast<const float*>(Wg),
                     static_cast<const float*>(Wu), I, static_cast<float*>(out), ld_out);
  return hipGetLastError();
}

}  // namespace tg
