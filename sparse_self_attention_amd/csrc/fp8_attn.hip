// FP8 value path for gfx950: V-Smooth quantisation of V and the sparse forward with ExpCast
// probabilities and an FP8 P.V product.
//
// What is computed (V-Smart/ExpCast summary, its V-Smooth and ExpCast-FP8 paragraphs):
//  * V-Smooth: per block of 128 tokens and channel the mean is subtracted (kept as bf16, 16 bits
//    per 128 elements) and the residual is quantised to E4M3 with one scale per channel; the
//    mean returns through the softmax row sums.  The channel scale is the power of two 2^e with
//    the smallest e such that 448 * 2^e covers the largest residual, so residual / scale and
//    mean / scale are exact.
//  * ExpCast: the probability byte is one multiply-add of the raw score plus an integer,
//    round-half-even(8 (x - m) + 120) clamped to [0, 126], where x is the score in log2 units and
//    m the row's reference point.  m lies on the 1/8 grid: ceil8(max) of the first block of 64
//    listed keys; a later block moves it only when one of its bytes would pass 126, and then by the
//    smallest whole number of log2 units that brings the block max to or below it.  The bias
//    120 = 56 + 64 carries the probability scaled by 2^8.
//
// Mapping onto CDNA4
// ------------------
//  * One workgroup per (batch, head, group); wave w owns query rows [32w, 32w+32).  Tiles of 64
//    listed keys: K rows (bf16), V rows (E4M3, D bytes) and one 32-byte slot row per key are
//    gathered into LDS with 16-byte buffer-load-to-LDS instructions, double-buffered.
//  * S^T = K Q^T with v_mfma_f32_32x32x16_bf16 as in the bf16 path (two 32-key halves); each lane
//    owns one query row and 32 of the 64 keys, and its 32 probability bytes are exactly the B
//    operand of v_mfma_f32_32x32x64_f8f6f4 for its row: no shuffle between the two products.
//    Byte b = 16 s + r of lane (row, h) holds key 32 s + 8 (r / 4) + 4 h + r % 4.
//  * The byte: y = fma(score, 8 scale log2e, 1.5 * 2^23 + 120 - 8m) puts round-half-even(8 (x - m)
//    + 120) in the low mantissa bits; an integer clamp to [0, 127] and v_perm_b32 pack four bytes
//    per word.  A byte of 127 flags the rare block whose reference point must move.
//  * Moves are whole powers of two, so O is never rescaled: O, the slot sums and the row sums stay
//    in the frame of the row's first reference point and each product takes its row's 2^(m - m0)
//    through the per-lane E8M0 B scale of v_mfma_scale_f32_32x32x64_f8f6f4 (exact).  The scale is
//    capped at 2^90 (the fp32 sums stay finite): a row whose max grows by more than 90 log2 units past
//    its first block would weigh its later blocks as if it had grown by 90, so its out and lse are
//    written as NaN instead.
//  * O^T += V8^T P^T: A = the V codes read from LDS with ds_read_b64_tr_b8 (the gfx950 transposing
//    byte read), four 8-byte reads per 64-key tile and 32 output dims.  Rows are XOR-swizzled in
//    32-byte pairs so the eight rows of one transposing read hit distinct banks.
//  * Block means: sum_j p_j mean_{b(j)} = sum_b L_b mean_b with L_b the row sum of p over the listed
//    keys of block b.  Blocks are grouped in aligned windows of 32; key j's slot is b(j) mod 32, and
//    its slot row (0x38 = E4M3 1.0 at byte b(j) mod 32) is copied from a 1 KB table by the same DMA,
//    so one more FP8 MFMA with A = the transposed slot rows accumulates L (32 slots x 32 rows) next
//    to O with no VALU work.  When the list passes into the next window, L is folded into O with
//    v_mfma_f32_32x32x16_bf16 (A = mean / scale of the window's blocks, channel-major in HBM; B = L
//    rounded to bf16) and the row sums take sum_b L_b.  A tile that straddles windows masks P per
//    window for the slot product.
#include <stdlib.h>

#include <type_traits>

#include "device_common.hpp"
#include "launch.hpp"

namespace sattn {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2v __attribute__((ext_vector_type(2)));

constexpr int VS_BLOCK = VSMOOTH_BLOCK;   // tokens per V-Smooth mean block
constexpr int F8_BK = 64;       // listed keys per tile
constexpr int F8_WIN = 32;      // mean blocks per slot window
constexpr int F8_MAX_GROWTH = 90;   // log2 units a row max may grow past its first block

// ---------------------------------------------------------------------------------------------
// V-Smooth quantisation
// ---------------------------------------------------------------------------------------------

// Nearest bf16 of a double, ties to even: truncate to fp32 with round-to-odd (sticky bit), then
// round fp32 -> bf16 to nearest even; round-to-odd with 16 spare bits makes the double rounding exact.
__device__ inline uint32_t bf16_bits_rne_f64(double x) {
  const float t = __double2float_rz(x);
  uint32_t u = __float_as_uint(t);
  if ((double)t != x) u |= 1u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Per (head, block): bf16 block means (exact fp64 sum of the bf16 tokens, divided by the token
// count) and the per-channel max |v - mean| of the block.  Thread t reads 16-byte pieces (8 channels)
// of every RPT-th token row; the fp64 sums are exact, so their order does not matter.
template <int D>
__global__ __launch_bounds__(256) void k_vs_stats(const uint16_t* __restrict__ v, int Nk, int NB,
                                                  uint16_t* __restrict__ mean_ws, float* __restrict__ bmax_ws) {
  constexpr int CG = D / 8;               // 16-byte channel groups per row
  constexpr int RPT = 256 / CG;           // token rows read at once
  constexpr int TOK = VS_BLOCK / RPT;     // tokens per thread
  __shared__ double part[RPT][D];
  __shared__ float pmax[RPT][D];
  __shared__ float meanf[D];
  const int blk = (int)(blockIdx.x % (uint32_t)NB);
  const size_t bh = blockIdx.x / (uint32_t)NB;
  const int cg = threadIdx.x % CG, tr = threadIdx.x / CG;
  const int nb0 = blk * VS_BLOCK;
  const int ntok = min(VS_BLOCK, Nk - nb0);
  const uint16_t* vb = v + (bh * Nk + nb0) * D + 8 * cg;
  u32x4 w[TOK];
#pragma unroll
  for (int i = 0; i < TOK; ++i) {
    const int t = tr + i * RPT;
    w[i] = t < ntok ? *(const u32x4*)(vb + (size_t)t * D) : u32x4{0u, 0u, 0u, 0u};
  }
  auto elem = [&](int i, int c) { return bf16_bits_to_float((w[i][c >> 1] >> (16 * (c & 1))) & 0xffffu); };
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    double s = 0.0;
#pragma unroll
    for (int i = 0; i < TOK; ++i) s += (double)elem(i, c);
    part[tr][8 * cg + c] = s;
  }
  __syncthreads();
  if (threadIdx.x < D) {
    const int d = threadIdx.x;
    double tot = 0.0;
#pragma unroll
    for (int r = 0; r < RPT; ++r) tot += part[r][d];
    const uint32_t mb = bf16_bits_rne_f64(tot / (double)ntok);
    meanf[d] = bf16_bits_to_float(mb);
    mean_ws[(bh * NB + blk) * D + d] = (uint16_t)mb;
  }
  __syncthreads();
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const float mf = meanf[8 * cg + c];
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < TOK; ++i)
      if (tr + i * RPT < ntok) m = fmaxf(m, fabsf(elem(i, c) - mf));
    pmax[tr][8 * cg + c] = m;
  }
  __syncthreads();
  if (threadIdx.x < D) {
    const int d = threadIdx.x;
    float a = pmax[0][d];
#pragma unroll
    for (int r = 1; r < RPT; ++r) a = fmaxf(a, pmax[r][d]);
    bmax_ws[(bh * NB + blk) * D + d] = a;
  }
}

// Per head: channel scale 2^e, the smallest power of two with 448 * 2^e >= max |residual|.  VS_SLICES
// threads per channel take every VS_SLICES-th block; the slice maxima meet in LDS.
constexpr int VS_SLICES = 8;
template <int D>
__global__ __launch_bounds__(D * VS_SLICES) void k_vs_scale(const float* __restrict__ bmax_ws, int NB,
                                                           float* __restrict__ vscale) {
  __shared__ float part[VS_SLICES][D];
  const size_t bh = blockIdx.x;
  const int d = threadIdx.x % D, sl = threadIdx.x / D;
  float a = 0.0f;
  for (int b = sl; b < NB; b += VS_SLICES) a = fmaxf(a, bmax_ws[(bh * NB + b) * D + d]);
  part[sl][d] = a;
  __syncthreads();
  if (sl != 0) return;
#pragma unroll
  for (int k = 1; k < VS_SLICES; ++k) a = fmaxf(a, part[k][d]);
  int e = 0;
  if (a > 0.0f) {
    int x;
    const float f = frexpf(a, &x);        // a = f 2^x, 0.5 <= f < 1; 448 = 0.875 * 2^9
    e = f <= 0.875f ? x - 9 : x - 8;
  }
  vscale[bh * D + d] = ldexpf(1.0f, e);
}

// Per (head, block): E4M3 codes of (v - mean) / scale and the channel-major scaled means.
template <int D>
__global__ __launch_bounds__(256) void k_vs_codes(const uint16_t* __restrict__ v, int Nk, int NB, int nbp,
                                                  const uint16_t* __restrict__ mean_ws,
                                                  const float* __restrict__ vscale, uint8_t* __restrict__ codes,
                                                  uint16_t* __restrict__ vmean) {
  constexpr int CH = D / 8;               // 16-byte chunks of a bf16 row
  __shared__ float mu[D], inv[D];
  const int blk = (int)(blockIdx.x % (uint32_t)NB);
  const size_t bh = blockIdx.x / (uint32_t)NB;
  const int nb0 = blk * VS_BLOCK;
  const int ntok = min(VS_BLOCK, Nk - nb0);
  if (threadIdx.x < D) {
    const int d = threadIdx.x;
    const float m = bf16_bits_to_float(mean_ws[(bh * NB + blk) * D + d]);
    const float is = 1.0f / vscale[bh * D + d];          // exact: the scale is a power of two
    mu[d] = m;
    inv[d] = is;
    uint16_t* mrow = vmean + (bh * D + d) * (size_t)nbp;
    mrow[blk] = (uint16_t)(__float_as_uint(m * is) >> 16);   // exact: bf16 times a power of two
    if (blk == NB - 1)
      for (int b = NB; b < nbp; ++b) mrow[b] = 0;
  }
  __syncthreads();
  for (int w = threadIdx.x; w < ntok * CH; w += 256) {
    const int t = w / CH, ch = w % CH;
    const size_t off = (bh * Nk + nb0 + t) * D + ch * 8;
    const u32x4 raw = *(const u32x4*)(v + off);
    float x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t bits = (raw[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
      x[i] = (bf16_bits_to_float(bits) - mu[ch * 8 + i]) * inv[ch * 8 + i];
    }
    uint32_t lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);
    lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], (int)lo, true);
    uint32_t hi = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x[4], x[5], 0, false);
    hi = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x[6], x[7], (int)hi, true);
    *(u32x2*)(codes + off) = u32x2{lo, hi};
  }
}

int launch_vsmooth(const VsmoothArgs& a) {
  const int NB = (a.Nk + VS_BLOCK - 1) / VS_BLOCK;
  const int nbp = vsmooth_mean_stride(a.Nk);
  const uint32_t BH = (uint32_t)a.B * (uint32_t)a.H;
  uint16_t* mean_ws = (uint16_t*)a.workspace;
  float* bmax_ws = (float*)((char*)a.workspace + vsmooth_mean_ws_bytes(a.B * a.H, a.Nk, a.D));
  hipStream_t st = (hipStream_t)a.stream;
  const uint16_t* v = (const uint16_t*)a.v;
  log_launch("k_vs_stats / k_vs_scale / k_vs_codes <D=%d>: %u x %d blocks of 128 tokens", a.D, BH, NB);
  if (a.D == 128) {
    hipLaunchKernelGGL(k_vs_stats<128>, dim3(BH * NB), dim3(256), 0, st, v, a.Nk, NB, mean_ws, bmax_ws);
    hipLaunchKernelGGL(k_vs_scale<128>, dim3(BH), dim3(128 * VS_SLICES), 0, st, bmax_ws, NB, a.vscale);
    hipLaunchKernelGGL(k_vs_codes<128>, dim3(BH * NB), dim3(256), 0, st, v, a.Nk, NB, nbp, mean_ws, a.vscale,
                       a.codes, (uint16_t*)a.vmean);
  } else {
    hipLaunchKernelGGL(k_vs_stats<64>, dim3(BH * NB), dim3(256), 0, st, v, a.Nk, NB, mean_ws, bmax_ws);
    hipLaunchKernelGGL(k_vs_scale<64>, dim3(BH), dim3(64 * VS_SLICES), 0, st, bmax_ws, NB, a.vscale);
    hipLaunchKernelGGL(k_vs_codes<64>, dim3(BH * NB), dim3(256), 0, st, v, a.Nk, NB, nbp, mean_ws, a.vscale,
                       a.codes, (uint16_t*)a.vmean);
  }
  return (int)hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// MXFP4 quantisation of queries and keys (4-bit QK^T)
// ---------------------------------------------------------------------------------------------

// Nearest E2M1 code of y (|y| <= 6), ties to the even code: the magnitude index counts the midpoints
// passed, strictly where the lower neighbour is even and inclusively where the upper one is.
__device__ inline uint32_t e2m1_code(float y) {
  const float a = fabsf(y);
  const uint32_t c = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) + (uint32_t)(a >= 1.75f) +
                     (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) + (uint32_t)(a > 5.0f);
  return y < 0.0f ? (c | 8u) : c;
}

// One thread per (row, block of 32): scale 2^e with the smallest e such that 6 * 2^e >= max |x|
// (at least 2^-127; 2^0 for a zero block), codes of x / 2^e packed two per byte (even element low).
// Scales take 4 bytes a row (byte b = block b; at D = 64 bytes 2 and 3 hold 127, i.e. 1.0).
template <int D>
__global__ __launch_bounds__(256) void k_mx4_quant(const uint16_t* __restrict__ x, uint32_t nrows,
                                                   uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  constexpr int NB = D / 32;
  const uint32_t t = blockIdx.x * 256u + threadIdx.x;
  if (t >= nrows * (uint32_t)NB) return;
  const uint32_t row = t / NB, b = t % NB;
  const u32x4* src = (const u32x4*)(x + (size_t)row * D + b * 32);
  float v[32];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u32x4 w = src[i];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[8 * i + j] = bf16_bits_to_float((w[j >> 1] >> (16 * (j & 1))) & 0xFFFFu);
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  int e = 0;
  if (amax > 0.0f) {
    int xe;
    const float f = frexpf(amax, &xe);    // amax = f 2^xe, 0.5 <= f < 1; 6 = 0.75 * 2^3
    e = max(f <= 0.75f ? xe - 3 : xe - 2, -127);
  }
  const float inv = ldexpf(1.0f, -e);     // exact: x / 2^e for bf16 x
  u32x4 out = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 32; ++i) out[i >> 3] |= e2m1_code(v[i] * inv) << (4 * (i & 7));
  *(u32x4*)(codes + (size_t)row * (D / 2) + b * 16) = out;
  scales[(size_t)row * 4 + b] = (uint8_t)(e + 127);
  if (NB == 2) scales[(size_t)row * 4 + 2 + b] = 127;
}

int launch_mx4_quant(const Mx4QuantArgs& a) {
  const uint32_t nrows = (uint32_t)a.B * (uint32_t)a.H * (uint32_t)a.N;
  const uint32_t threads = nrows * (uint32_t)(a.D / 32);
  const dim3 grid((threads + 255) / 256);
  hipStream_t st = (hipStream_t)a.stream;
  log_launch("k_mx4_quant<D=%d>: %u rows, %u workgroups x 256 threads", a.D, nrows, grid.x);
  if (a.D == 128)
    hipLaunchKernelGGL(k_mx4_quant<128>, grid, dim3(256), 0, st, (const uint16_t*)a.x, nrows, a.codes, a.scales);
  else
    hipLaunchKernelGGL(k_mx4_quant<64>, grid, dim3(256), 0, st, (const uint16_t*)a.x, nrows, a.codes, a.scales);
  return (int)hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Sparse forward with ExpCast bytes and the FP8 P.V product
// ---------------------------------------------------------------------------------------------

template <int D, bool QK4 = false>
struct F8Layout {
  // K rows in LDS: bf16 (2D bytes), or E2M1 codes (D/2 bytes) followed by a region of per-key E8M0
  // scales (D/32 bytes per key) for the 4-bit product
  static constexpr int RB = QK4 ? D / 2 : 2 * D;
  static constexpr int NC = RB / 16;               // 16-byte chunks per K row
  static constexpr int RPL = 1024 / RB;            // K rows filled by one 64-lane 16-byte load
  static constexpr int KSETS = F8_BK / RPL;        // K loads per tile
  static constexpr int KSB = 4;                    // scale bytes per row (4-bit product; D / 32 used)
  static constexpr int NC8 = D / 16;               // 16-byte chunks per E4M3 V row
  static constexpr int RPL8 = 1024 / D;            // V rows per load
  static constexpr int VSETS = F8_BK / RPL8;       // V loads per tile
  static constexpr int KBYTES = F8_BK * RB + (QK4 ? 1024 : 0);   // codes + scale region (1 KB aligned)
  static constexpr int KSOFF = F8_BK * RB;                      // offset of the scale region
  static constexpr int VBYTES = F8_BK * D;
  static constexpr int IBYTES = F8_BK * 32;        // one 32-byte slot row per key
  static constexpr int STAGE = KBYTES + VBYTES + IBYTES;
  static constexpr int KSTEPS = D / 16;
  static constexpr int DBLK = D / 32;
  static constexpr int ROWDIV = QK4 ? 4 : 16 / NC;
  // register budget: two waves per SIMD at D = 128 (O, both score halves, Q and the slot sums
  // stay in VGPRs), three at D = 64
  static constexpr int WAVES_PER_EU = D == 128 ? 2 : 3;
  // bf16 K: 16 rows read at one chunk hit distinct banks; E2M1 K (64- or 32-byte rows read 16 bytes a
  // lane): rows r and r + 4 of a 64-byte-row tile trade chunks
  __device__ static inline int swz_k(int row) { return (row / ROWDIV) % NC; }
  // 32-byte pair of a V row: the transposing read takes rows {0,1,2,3,8,9,10,11} (+4h, +16t) at one
  // pair index; this XOR spreads them over all 64 banks
  __device__ static inline int swz_v(int row) {
    return D == 128 ? (((row >> 1) & 1) | (((row >> 3) & 1) << 1)) : ((row >> 3) & 1);
  }
};

template <int N>
using F8IC = std::integral_constant<int, N>;

// Slot rows: row m holds E4M3 1.0 (0x38) at byte m and zeros elsewhere.
struct OneHotTable {
  uint8_t b[F8_WIN * 32];
};
constexpr OneHotTable make_onehot() {
  OneHotTable t{};
  for (int m = 0; m < F8_WIN; ++m) t.b[m * 32 + m] = 0x38;
  return t;
}
__device__ __attribute__((aligned(256))) const OneHotTable k_onehot = make_onehot();

// Stored position of slot row r of a tile: rows 8..11 and 12..15 of every 16 trade places, so the
// eight rows one transposing read touches ({0..3, 8..11} + 4h) cover all 64 banks.  An involution.
__device__ inline int ind_pos(int r) { return r ^ ((r & 8) >> 1); }

// The lane id from v_mbcnt, behind an asm barrier so the compiler cannot hoist it out of a loop into a
// register that lives (and may be spilled) across the loop.
__device__ inline int opaque_lane_id() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// ExpCast: the float bits clamped so that the low byte is the code, 0..127 (0x4B400000 = 1.5 * 2^23
// holds 0; 127 flags a byte past the largest finite code)
__device__ inline uint32_t expcast_bits(float s, float c1, float c0) {
  const int y = (int)__float_as_uint(__builtin_fmaf(s, c1, c0));
  return (uint32_t)min(max(y, 0x4B400000), 0x4B40007F);
}
// low bytes of four words -> one word (v_perm_b32: selector bytes 0-3 pick from the second operand,
// 4-7 from the first, 0x0C gives 0)
__device__ inline uint32_t pack4(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const uint32_t ab = __builtin_amdgcn_perm(b, a, 0x0C0C0400u);
  const uint32_t cd = __builtin_amdgcn_perm(d, c, 0x0C0C0400u);
  return __builtin_amdgcn_perm(cd, ab, 0x05040100u);
}
// byte masks of the keys [lo, hi) of a tile for the four keys 8 w + 4 h + 0..3 of dword w
__device__ inline uint32_t key_byte_mask(uint64_t m64, int w, int h) {
  const uint32_t nib = (uint32_t)(m64 >> (8 * w + 4 * h)) & 0xFu;
  const uint32_t spread = (nib * 0x00204081u) & 0x01010101u;
  return (spread << 8) - spread;
}

// QK4: Q and K arrive as E2M1 codes (D/2 bytes a row) with E8M0 scales per 32 elements (qs, ks) and the
// scores come from v_mfma_scale_f32_32x32x64_f8f6f4 in FP4 x FP4, two products per 32-key half at D = 128.
template <int D, int NW, bool OUT_F32, bool QK4>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(F8Layout<D, QK4>::WAVES_PER_EU,
                                                                         F8Layout<D, QK4>::WAVES_PER_EU))) void attn_fwd_fp8(
    const void* __restrict__ qv, const void* __restrict__ kv, const uint8_t* __restrict__ qs,
    const uint8_t* __restrict__ ks, const uint8_t* __restrict__ v8,
    const float* __restrict__ vscale, const uint16_t* __restrict__ vmean, int nbp,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ counts, int cap, int Nq, int Nk, int group, int G,
    float scale_log2, void* __restrict__ out, float* __restrict__ lse, uint32_t n_units, int row0) {
  using L = F8Layout<D, QK4>;
  constexpr int NKS = (L::KSETS + NW - 1) / NW;
  constexpr int NVS = (L::VSETS + NW - 1) / NW;
  constexpr int ISETS = L::IBYTES / 1024;          // slot-row loads per tile (2)
  static_assert(NW >= ISETS, "one slot-row load per wave");
  // Each stage's K, V and slot-row tiles are LDS objects of their own, so the compiler can tell that the
  // reads of one stage do not depend on the gather in flight into the other one (no wait for it).
  __shared__ __attribute__((aligned(1024))) char sk0[L::KBYTES];
  __shared__ __attribute__((aligned(1024))) char sv0[L::VBYTES];
  __shared__ __attribute__((aligned(1024))) char si0[L::IBYTES];
  __shared__ __attribute__((aligned(1024))) char sk1[L::KBYTES];
  __shared__ __attribute__((aligned(1024))) char sv1[L::VBYTES];
  __shared__ __attribute__((aligned(1024))) char si1[L::IBYTES];

  const uint32_t unit = xcd_striped(blockIdx.x, n_units, 128);
  const int g = (int)(unit % (uint32_t)G);
  const uint32_t bh = unit / (uint32_t)G;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hi = lane >> 5;
  const int ql = lane & 31;
  // this launch covers rows [row0, row0 + 32 NW) of the group (wider groups run as several launches)
  const int r0 = g * group + row0;
  const int rows_here = min(min(group - row0, NW * 32), Nq - r0);
  if (rows_here <= 0) return;   // the partial last group may end before this launch's rows
  const int wrow = wave * 32 + ql;
  const bool row_valid = wrow < rows_here;

  int c = counts[bh * (uint32_t)G + g];
  c = c < 0 ? 0 : (c > cap ? cap : c);
  const int nblk = (c + F8_BK - 1) / F8_BK;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc((const char*)kv + (size_t)bh * Nk * L::RB, (uint32_t)Nk * L::RB);
  const __amdgpu_buffer_rsrc_t rks =
      make_rsrc(QK4 ? ks + (size_t)bh * Nk * L::KSB : nullptr, QK4 ? (uint32_t)Nk * L::KSB : 0u);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(v8 + (size_t)bh * Nk * D, (uint32_t)Nk * D);
  const __amdgpu_buffer_rsrc_t rm = make_rsrc(vmean + (size_t)bh * D * nbp, (uint32_t)(D * nbp * 2));
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(k_onehot.b, (uint32_t)sizeof(k_onehot.b));
  const int32_t* ilist = idx + ((size_t)bh * G + g) * (size_t)cap;
  // the list through a buffer resource: 32-bit offsets, no 64-bit address arithmetic per load
  const __amdgpu_buffer_rsrc_t ri = make_rsrc(ilist, (uint32_t)c * 4u);
  auto list_at = [&](int p) { return (int)__builtin_amdgcn_raw_buffer_load_b32(ri, (uint32_t)min(p, c - 1) * 4u, 0, 0); };

  // the wave's query rows: bf16 (8 k-steps of 16 dims) or E2M1 (D/64 steps of 64 dims, 16 bytes a lane)
  constexpr int QREGS = QK4 ? D / 64 : L::KSTEPS;
  u32x4 qf[QREGS];
  uint32_t qscale = 0;     // E8M0 scales of the lane's blocks 2t + hi, in byte 2t after the shift
  {
    const __amdgpu_buffer_rsrc_t rq = make_rsrc((const char*)qv + (size_t)bh * Nq * L::RB, (uint32_t)Nq * L::RB);
    const uint32_t rowoff = row_valid ? (uint32_t)(r0 + wrow) * L::RB : (uint32_t)Nq * L::RB;
#pragma unroll
    for (int t = 0; t < QREGS; ++t) qf[t] = buffer_load_x4(rq, rowoff + (uint32_t)(2 * t + hi) * 16);
    if constexpr (QK4) {
      const uint8_t* qsr = qs + ((size_t)bh * Nq + r0 + (row_valid ? wrow : 0)) * L::KSB;
      qscale = *(const uint32_t*)qsr >> (8 * hi);
    }
  }
  // per-lane offsets are recomputed where used (a few integer operations) rather than held in VGPRs
  const uint32_t kbase = ql * L::RB;
  const int kswz = L::swz_k(ql);
  auto koff = [&](int ks) { return kbase + 16u * (uint32_t)((2 * ks + hi) ^ kswz); };
  // transposing reads: lane j of each 16-lane group supplies row vrow (+16 t) at byte 8 (j % 2) of
  // the 16-byte chunk 2 db + (group % 2) (V codes) or (group % 2) (slot rows)
  const int j16 = lane & 15, g16 = lane >> 4;
  const int e8 = j16 >> 1;
  const int vrow = 8 * (e8 >> 2) + 4 * hi + (e8 & 3);
  const uint32_t vbase = vrow * D + 16 * (g16 & 1) + 8 * (j16 & 1);
  const int vswz = L::swz_v(vrow);
  auto voff = [&](int db) { return vbase + 32u * (uint32_t)(db ^ vswz); };
  const uint32_t ioff = ind_pos(vrow) * 32 + 16 * (g16 & 1) + 8 * (j16 & 1);

  const int krow_in = lane / L::NC, kpos = lane % L::NC;
  const int vrow_in = lane / L::NC8, vpos = lane % L::NC8;
  auto kch = [&](int j) {
    const int row = (wave + j * NW) * L::RPL + krow_in;
    return 16u * (uint32_t)(kpos ^ L::swz_k(row));
  };
  auto vch = [&](int j) {
    const int row = (wave + j * NW) * L::RPL8 + vrow_in;
    return 16u * (uint32_t)(2 * ((vpos >> 1) ^ L::swz_v(row)) + (vpos & 1));
  };
  // slot-row load of this wave (waves 0 and 1): LDS position 32 wave + lane / 2 holds key row
  // ind_pos(position), chunk lane % 2.  The row is recomputed from the lane id at each fetch: held across
  // the loop it would be spilled, and its reload right after the gather is issued waits for that gather.
  auto irow = [&]() { return ind_pos(32 * wave + (opaque_lane_id() >> 1)); };
  int kkeys[NKS], vkeys[NVS], ikey = 0, skey = 0;
  const int swave = NW - 1;        // the wave that gathers the keys' E8M0 scales (4-bit product)
  // The lane's row within a load.  In the variants whose registers overflow (FP8 scores of three waves,
  // 4-bit scores at D = 64 with three or four waves) it is recomputed from the lane id at each fetch:
  // held across the loop it is spilled, and its reload right after the gather is issued waits for that
  // gather (FP8 scores on the voxel workload's 96-row slices: 13.8 -> 8.4 ms).  Elsewhere it stays in a
  // register (the recompute's scheduling barrier costs 1-4 % there).
  constexpr bool RECOMPUTE_ROWS = QK4 ? (D == 64 && NW >= 3) : NW == 3;
  auto fetch_keys = [&](int blk) {
    if constexpr (RECOMPUTE_ROWS) {
      const int lid = opaque_lane_id();
#pragma unroll
      for (int j = 0; j < NKS; ++j) {
        const int rs = wave + j * NW;
        const int p = blk * F8_BK + rs * L::RPL + lid / L::NC;
        if (L::KSETS % NW == 0 || rs < L::KSETS) kkeys[j] = list_at(p);
      }
#pragma unroll
      for (int j = 0; j < NVS; ++j) {
        const int rs = wave + j * NW;
        const int p = blk * F8_BK + rs * L::RPL8 + lid / L::NC8;
        if (L::VSETS % NW == 0 || rs < L::VSETS) vkeys[j] = list_at(p);
      }
    } else {
#pragma unroll
      for (int j = 0; j < NKS; ++j) {
        const int rs = wave + j * NW;
        const int p = blk * F8_BK + rs * L::RPL + krow_in;
        if (L::KSETS % NW == 0 || rs < L::KSETS) kkeys[j] = list_at(p);
      }
#pragma unroll
      for (int j = 0; j < NVS; ++j) {
        const int rs = wave + j * NW;
        const int p = blk * F8_BK + rs * L::RPL8 + vrow_in;
        if (L::VSETS % NW == 0 || rs < L::VSETS) vkeys[j] = list_at(p);
      }
    }
    if (wave < ISETS) {
      const int p = blk * F8_BK + irow();
      ikey = list_at(p);
    }
    if (QK4 && wave == swave) {
      const int p = blk * F8_BK + lane;
      skey = list_at(p);
    }
  };
  // gathered indices are clamped to Nk: any out-of-range list value reads the zero row past the buffer end
  auto issue = [&](char* kst, char* vst, char* ist) {
#pragma unroll
    for (int j = 0; j < NKS; ++j) {
      const int rs = wave + j * NW;
      if (L::KSETS % NW == 0 || rs < L::KSETS)
        buffer_load_lds_x4(rk, kst + rs * L::RPL * L::RB, min((uint32_t)kkeys[j], (uint32_t)Nk) * L::RB + kch(j));
    }
#pragma unroll
    for (int j = 0; j < NVS; ++j) {
      const int rs = wave + j * NW;
      if (L::VSETS % NW == 0 || rs < L::VSETS)
        buffer_load_lds_x4(rv, vst + rs * L::RPL8 * D, min((uint32_t)vkeys[j], (uint32_t)Nk) * D + vch(j));
    }
    if (wave < ISETS)
      buffer_load_lds_x4(ro, ist + wave * 1024,
                         (uint32_t)((ikey >> 7) & (F8_WIN - 1)) * 32u + 16u * (uint32_t)(lane & 1));
    if (QK4 && wave == swave)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rks, SATTN_LDS_PTR(void, kst + L::KSOFF), L::KSB,
                                               min((uint32_t)skey, (uint32_t)Nk) * L::KSB, 0, 0, 0);
  };
  // the tile's listed key of this lane (lane = position in the tile), for the mean windows
  auto tile_key = [&](int blk) {
    const int p = blk * F8_BK + lane;
    return p < c ? list_at(p) : -1;
  };

  f32x16 o[L::DBLK];
#pragma unroll
  for (int i = 0; i < L::DBLK; ++i) o[i] = f32x16{};
  f32x16 lb = {};
  float m8 = 0.0f, mbase8 = 0.0f, l_run = 0.0f;
  int escale = 127;                 // E8M0 B scale of this row: 2^(m - m0)
  int win = 0, slot_lo = F8_WIN, slot_hi = -1;   // current window of 32 blocks; slots it has used
  const float c1 = scale_log2 * 8.0f;
  int tkey = 0;

  // fold the window's block means into O: O += (mean / scale)^T L, row sums += sum of L
  auto flush = [&]() {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      if ((ks == 0 && slot_lo >= 16) || (ks == 1 && slot_hi < 16)) continue;
      const u32x4 bw = {pack_bf16x2(lb[8 * ks], lb[8 * ks + 1]), pack_bf16x2(lb[8 * ks + 2], lb[8 * ks + 3]),
                        pack_bf16x2(lb[8 * ks + 4], lb[8 * ks + 5]), pack_bf16x2(lb[8 * ks + 6], lb[8 * ks + 7])};
#pragma unroll
      for (int db = 0; db < L::DBLK; ++db) {
        const uint32_t off =
            ((uint32_t)(32 * db + ql) * (uint32_t)nbp + (uint32_t)(F8_WIN * win + 16 * ks + 4 * hi)) * 2u;
        const u32x2 m0 = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rm, off, 0, 0));
        const u32x2 m1 = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rm, off + 16, 0, 0));
        const u32x4 aw = {m0[0], m0[1], m1[0], m1[1]};
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, aw), __builtin_bit_cast(bf16x8, bw),
                                                       o[db], 0, 0, 0);
      }
    }
    float s = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) s += lb[r];
    l_run += s;
    lb = f32x16{};
    slot_lo = F8_WIN;
    slot_hi = -1;
  };

  auto block = [&](auto st, int j) {
    constexpr int ST = decltype(st)::value;
    wait_vmcnt0();
    __syncthreads();
    const int key_here = tkey;
    if (j + 1 < nblk) {
      if (ST == 0) issue(sk1, sv1, si1);
      else issue(sk0, sv0, si0);
      if (j + 2 < nblk) fetch_keys(j + 2);
      tkey = tile_key(j + 1);
    }
    const char* sk = ST == 0 ? sk0 : sk1;
    const char* sv = ST == 0 ? sv0 : sv1;
    const char* si = ST == 0 ? si0 : si1;
    f32x16 s0 = {}, s1 = {};
    if constexpr (QK4) {
      // E8M0 scales of keys ql and 32 + ql, shifted so byte 2t holds block 2t + hi
      const char* sks = sk + L::KSOFF;
      const uint32_t k0s = *(const uint32_t*)(sks + ql * 4) >> (8 * hi);
      const uint32_t k1s = *(const uint32_t*)(sks + (32 + ql) * 4) >> (8 * hi);
      // one k-step of 64 dims; the scale byte select (2t) must be an immediate
      auto kstep = [&](auto tc) {
        constexpr int t = decltype(tc)::value;
        const u32x4 a0 = *(const u32x4*)(sk + koff(t));
        const u32x4 a1 = *(const u32x4*)(sk + 32 * L::RB + koff(t));
        const i32x8 b8 = {(int)qf[t][0], (int)qf[t][1], (int)qf[t][2], (int)qf[t][3], 0, 0, 0, 0};
        const i32x8 a08 = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], 0, 0, 0, 0};
        const i32x8 a18 = {(int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3], 0, 0, 0, 0};
        s0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a08, b8, s0, 4, 4, 2 * t, (int)k0s, 2 * t, (int)qscale);
        s1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a18, b8, s1, 4, 4, 2 * t, (int)k1s, 2 * t, (int)qscale);
      };
      kstep(F8IC<0>{});
      if constexpr (QREGS > 1) kstep(F8IC<1>{});
    } else {
#pragma unroll
      for (int ks = 0; ks < L::KSTEPS; ++ks) {
        const bf16x8 a0 = *(const bf16x8*)(sk + koff(ks));
        const bf16x8 a1 = *(const bf16x8*)(sk + 32 * L::RB + koff(ks));
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, __builtin_bit_cast(bf16x8, qf[ks]), s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, __builtin_bit_cast(bf16x8, qf[ks]), s1, 0, 0, 0);
      }
    }
    const int valid = min(F8_BK, c - j * F8_BK);
    if (valid < F8_BK) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kk = 8 * (r >> 2) + 4 * hi + (r & 3);
        if (kk >= valid) s0[r] = -INFINITY;
        if (kk + 32 >= valid) s1[r] = -INFINITY;
      }
    }
    auto block_max = [&]() {
      float bmax = fmaxf(s0[0], s1[0]);
#pragma unroll
      for (int r = 1; r < 16; ++r) bmax = fmaxf(bmax, fmaxf(s0[r], s1[r]));
      return pair_max(bmax) * scale_log2;
    };
    // ExpCast bytes, already in the B-operand order of the FP8 products
    i32x8 pb;
    auto make_bytes = [&]() {
      const float c0 = 12582912.0f + 120.0f - m8;
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const int r = 4 * (w & 3);
        const float x0 = w < 4 ? s0[r] : s1[r], x1 = w < 4 ? s0[r + 1] : s1[r + 1];
        const float x2 = w < 4 ? s0[r + 2] : s1[r + 2], x3 = w < 4 ? s0[r + 3] : s1[r + 3];
        pb[w] = (int)pack4(expcast_bits(x0, c1, c0), expcast_bits(x1, c1, c0), expcast_bits(x2, c1, c0),
                           expcast_bits(x3, c1, c0));
      }
    };
    if (j == 0) {
      m8 = ceilf(8.0f * block_max());
      mbase8 = m8;
      make_bytes();
    } else {
      make_bytes();
      uint32_t acc = 0;
#pragma unroll
      for (int w = 0; w < 8; ++w) acc |= (uint32_t)pb[w] + 0x01010101u;
      // a byte of 127 (past the largest finite code) in either lane of the row moves the row's point
      const uint64_t mv = __builtin_amdgcn_ballot_w64((acc & 0x80808080u) != 0);
      if (mv != 0) {
        const bool move = ((mv >> ql) | (mv >> (ql + 32))) & 1u;
        const float bmax = block_max();
        if (move) m8 += 8.0f * ceilf(bmax - m8 * 0.125f);
        make_bytes();
        // the frame holds 2^90 of growth past the first block (fp32 sums of up to 2^11 tiles stay finite)
        escale = 127 + min((int)((m8 - mbase8) * 0.125f), F8_MAX_GROWTH);
      }
    }
#pragma unroll
    for (int db = 0; db < L::DBLK; ++db) {
      const char* p0 = sv + voff(db);
      const i32x2v t0 = __builtin_amdgcn_ds_read_tr8_b64_v2i32(SATTN_LDS_PTR(i32x2v, p0));
      const i32x2v t1 = __builtin_amdgcn_ds_read_tr8_b64_v2i32(SATTN_LDS_PTR(i32x2v, p0 + 16 * D));
      const i32x2v t2 = __builtin_amdgcn_ds_read_tr8_b64_v2i32(SATTN_LDS_PTR(i32x2v, p0 + 32 * D));
      const i32x2v t3 = __builtin_amdgcn_ds_read_tr8_b64_v2i32(SATTN_LDS_PTR(i32x2v, p0 + 48 * D));
      const i32x8 av = {t0[0], t0[1], t1[0], t1[1], t2[0], t2[1], t3[0], t3[1]};
      o[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, pb, o[db], 0, 0, 0, 127, 0, escale);
    }
    i32x8 ia;
    {
      const char* p0 = si + ioff;
      const i32x2v t0 = __builtin_amdgcn_ds_read_tr8_b64_v2i32(SATTN_LDS_PTR(i32x2v, p0));
      const i32x2v t1 = __builtin_amdgcn_ds_read_tr8_b64_v2i32(SATTN_LDS_PTR(i32x2v, p0 + 512));
      const i32x2v t2 = __builtin_amdgcn_ds_read_tr8_b64_v2i32(SATTN_LDS_PTR(i32x2v, p0 + 1024));
      const i32x2v t3 = __builtin_amdgcn_ds_read_tr8_b64_v2i32(SATTN_LDS_PTR(i32x2v, p0 + 1536));
      ia = i32x8{t0[0], t0[1], t1[0], t1[1], t2[0], t2[1], t3[0], t3[1]};
    }
    // block-mean slot sums: this tile's keys by aligned window of 32 blocks (key >> 12)
    const int kw = key_here >= 0 ? (key_here >> 12) : 0x7FFFFFFF;
    const int kslot = (key_here >> 7) & (F8_WIN - 1);
    if (j == 0) win = __builtin_amdgcn_readfirstlane(kw);
    // keys of windows <= win form a prefix of the tile; a tile that straddles windows masks P to
    // each window's keys in turn (the common tile takes one pass with P unmasked)
    int lo = 0;
    while (true) {
      const int nhi = __builtin_popcountll(__builtin_amdgcn_ballot_w64(kw <= win));
      if (nhi > lo) {
        i32x8 pm = pb;
        if (lo > 0 || nhi < valid) {
          const uint64_t m64 = (nhi >= 64 ? ~0ull : ((1ull << nhi) - 1ull)) & ~((1ull << lo) - 1ull);
#pragma unroll
          for (int w = 0; w < 8; ++w) pm[w] = (int)((uint32_t)pb[w] & key_byte_mask(m64, w, hi));
        }
        lb = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ia, pm, lb, 0, 0, 0, 127, 0, escale);
        slot_lo = min(slot_lo, __builtin_amdgcn_readlane(kslot, lo));
        slot_hi = max(slot_hi, __builtin_amdgcn_readlane(kslot, nhi - 1));
      }
      if (nhi >= valid) break;
      flush();
      win = __builtin_amdgcn_readlane(kw, nhi);
      lo = nhi;
    }
  };

  if (nblk > 0) {
    fetch_keys(0);
    issue(sk0, sv0, si0);
    if (nblk > 1) fetch_keys(1);
    tkey = tile_key(0);
  }
  int j = 0;
  for (; j + 1 < nblk; j += 2) {
    block(F8IC<0>{}, j);
    block(F8IC<1>{}, j + 1);
  }
  if (j < nblk) block(F8IC<0>{}, j);
  if (nblk > 0) flush();

  const float l_tot = pair_sum(l_run);
  // a row whose point grew past the frame's range (F8_MAX_GROWTH) has weighed its later keys wrongly:
  // its out and lse are NaN rather than a wrong number
  const bool over_range = (m8 - mbase8) * 0.125f > (float)F8_MAX_GROWTH;
  const float inv = over_range ? __builtin_nanf("") : (l_tot > 0.0f ? 1.0f / l_tot : 0.0f);
  if (row_valid) {
    const size_t orow = ((size_t)bh * Nq + r0 + wrow) * D;
    const float* sc = vscale + (size_t)bh * D;
#pragma unroll
    for (int db = 0; db < L::DBLK; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d0 = 32 * db + 8 * i + 4 * hi;
        const f32x4 s = *(const f32x4*)(sc + d0);
        const float x0 = o[db][4 * i] * s[0] * inv, x1 = o[db][4 * i + 1] * s[1] * inv;
        const float x2 = o[db][4 * i + 2] * s[2] * inv, x3 = o[db][4 * i + 3] * s[3] * inv;
        if (OUT_F32) *(f32x4*)((float*)out + orow + d0) = f32x4{x0, x1, x2, x3};
        else *(u32x2*)((uint16_t*)out + orow + d0) = u32x2{pack_bf16x2(x0, x1), pack_bf16x2(x2, x3)};
      }
    if (lse != nullptr && hi == 0)
      lse[(size_t)bh * Nq + r0 + wrow] =
          over_range ? __builtin_nanf("")
                     : l_tot > 0.0f ? (mbase8 * 0.125f - 8.0f + __log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
  }
}

template <int D, int NW, bool QK4>
static int launch_fp8_t(const Fp8FwdArgs& a, int row0) {
  const uint32_t G = (uint32_t)((a.Nq + a.group - 1) / a.group);
  const uint32_t n_units = (uint32_t)a.B * (uint32_t)a.H * G;
  const float scale_log2 = a.scale * 1.4426950408889634f;
  const int nbp = vsmooth_mean_stride(a.Nk);
  hipStream_t st = (hipStream_t)a.stream;
  log_launch("attn_fwd_fp8<D=%d, waves=%d, %s, %s> rows %d.. of each group: %u workgroups x %d threads", D, NW,
             QK4 ? "MXFP4 scores" : "bf16 scores", a.out_f32 ? "f32" : "bf16", row0, n_units, NW * 64);
  if (a.out_f32)
    hipLaunchKernelGGL((attn_fwd_fp8<D, NW, true, QK4>), dim3(n_units), dim3(NW * 64), 0, st, a.q, a.k, a.q_scales,
                       a.k_scales, a.codes, a.vscale, (const uint16_t*)a.vmean, nbp, a.idx, a.counts, a.cap, a.Nq,
                       a.Nk, a.group, (int)G, scale_log2, a.out, a.lse, n_units, row0);
  else
    hipLaunchKernelGGL((attn_fwd_fp8<D, NW, false, QK4>), dim3(n_units), dim3(NW * 64), 0, st, a.q, a.k, a.q_scales,
                       a.k_scales, a.codes, a.vscale, (const uint16_t*)a.vmean, nbp, a.idx, a.counts, a.cap, a.Nq,
                       a.Nk, a.group, (int)G, scale_log2, a.out, a.lse, n_units, row0);
  return (int)hipGetLastError();
}

// Groups wider than 128 rows run as slices of 128 rows and a remainder, one launch per slice (a six- or
// eight-wave workgroup leaves most SIMDs of its CU under-filled).  Unlike the bf16 forward's equal
// slices (192 -> 2 x 96), this kernel holds two waves per SIMD, so four-wave workgroups fill a CU exactly
// (two of them) where three-wave ones leave 1.5 waves per SIMD: 192 -> 128 + 64 ran the FP8 forward on the
// voxel workload in 6.71 instead of 8.29 ms and the 4-bit score forward in 4.45 instead of 5.71 ms.
template <int D, bool QK4>
static int launch_fp8_d(const Fp8FwdArgs& a) {
  for (int row0 = 0; row0 < a.group; row0 += 128) {
    const int waves = (min(128, a.group - row0) + 31) / 32;
    const int err = waves <= 2 ? launch_fp8_t<D, 2, QK4>(a, row0)
                  : waves == 3 ? launch_fp8_t<D, 3, QK4>(a, row0) : launch_fp8_t<D, 4, QK4>(a, row0);
    if (err) return err;
  }
  return 0;
}

int launch_fp8_fwd(const Fp8FwdArgs& a) {
  const bool qk4 = a.q_scales != nullptr;
  if (a.D == 64) return qk4 ? launch_fp8_d<64, true>(a) : launch_fp8_d<64, false>(a);
  return qk4 ? launch_fp8_d<128, true>(a) : launch_fp8_d<128, false>(a);
}

}  // namespace sattn
