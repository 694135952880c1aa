// Fine-grained sparse attention forward (and the dense control path) for gfx950.
//
// What is computed (FG-Attn review, "What carries the argument", Fig. 6 and Fig. 7 captions;
// Chipmunk review, Referee major comment 1): every group of `group` contiguous queries attends
// only to the keys of its index list, with the softmax renormalised over those keys.
// The online softmax keeps a running max, a running sum of exponentials and a running output
// per query row and rescales them when the max grows (LongLive DiT blog, "Online Softmax").
//
// Mapping onto CDNA4
// ------------------
//  * One workgroup per (batch, head, group); wave w owns query rows [32w, 32w+32) of the group.  A
//    group wider than 128 rows runs as equal slices of at most 128 rows, one launch per slice.
//    Workgroup ids are striped over the XCDs in runs of 128 units, so the eight XCDs work on
//    neighbouring groups of one head at a time (its K/V stay in the last-level cache).
//  * Key blocks of 32 kept keys.  The block's K and V rows are gathered from HBM straight
//    into LDS with 16-byte buffer-load-to-LDS instructions (one lane = one 16 B chunk of a row),
//    double-buffered so the gather of block j+1 overlaps the math of block j.  Buffer loads
//    return zeros for an out-of-range row instead of faulting.
//  * Scores are produced transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: A = K rows
//    read from LDS, B = the wave's 32 query rows held in VGPRs for the whole loop.  In the
//    accumulator layout each lane then owns one query (lane % 32) and 16 of every 32 keys, so
//    the row max / row sum of the softmax are in-lane plus one lane-pair exchange.
//  * O^T = V^T P^T: B = the bf16 probabilities straight from the score accumulators, A = V^T
//    read from LDS with ds_read_b64_tr_b16 (the gfx950 transposing LDS read), so the output
//    accumulators also have one query per lane and the rescale by exp(m_old - m_new) is a
//    per-lane multiply.
//  * The softmax runs in base 2 with log2(e) folded into the score scale.  The running max is
//    taken from the first block and moved only when a later block has a probability above 2^64
//    (or an overflow), checked on the packed bf16 probabilities with integer maxima, so the common
//    path has no max reduction and no rescale.  P enters the PV product rounded to bf16, and the row
//    sum adds those same rounded values, so the output is exactly their weighted mean of V: with the
//    max taken lazily the dominant probability is not 1, and summing the fp32 values instead would
//    pass its rounding error (up to 2^-8 of it) straight into the output.
//  * The row sums run on the matrix cores: a 16x16x32 product of the probability registers with a
//    0/1 selector per block, which takes the ~30 fp32 VALU operations of an adder tree off the SIMDs
//    that also issue the exponentials.
//  * LDS rows are XOR-swizzled in 16-byte chunks: K rows so that 16 consecutive rows read at
//    the same chunk hit distinct banks, V rows so that the 4-row transposed reads do.
#include <stdlib.h>

#include <type_traits>

#include "device_common.hpp"
#include "launch.hpp"

namespace sattn {

// The running max is kept until a probability passes 2^64: the bf16 bit pattern of 2^64 (positive
// bf16 values order like their bit patterns).
constexpr uint32_t RESCALE_BF16_BITS = 0x5F80u;

template <int D, int BKEYS>
struct FwdLayout {
  static constexpr int RB = D * 2;                    // bytes per K/V row
  static constexpr int NC = D / 8;                    // 16-byte chunks per row
  static constexpr int ROWS_PER_LOAD = 1024 / RB;     // rows filled by one 64-lane 16-byte load
  static constexpr int ROWSETS = BKEYS / ROWS_PER_LOAD;  // load instructions per K (or V) block
  static constexpr int MAT_BYTES = BKEYS * RB;
  static constexpr int KSTEPS = D / 16;               // MFMA k-steps over the head dim
  static constexpr int DBLK = D / 32;                 // 32-wide output column blocks
  static constexpr int ROWDIV = 16 / NC;              // rows sharing one 256-byte bank sweep
  __device__ static inline int swz_k(int row) { return (row / ROWDIV) % NC; }
  __device__ static inline int swz_v(int row) { return 4 * ((row / ROWDIV) % (NC / 4)); }
};

template <int N>
using IC = std::integral_constant<int, N>;

// Lean variant: blocks of 32 kept keys, K+V double-buffered (32 KB of LDS at D = 128) and no
// cross-block register pipeline, so three workgroups (12 waves) fit per CU and the SIMDs
// interleave MFMA and softmax work of different waves.
constexpr int BKL = 32;

// DELTA: the Chipmunk sparse-delta update instead of the softmax.  The probabilities use the given
// (stale) lse instead of a running max and are not renormalised; the epilogue forms
// out = out_prev - fresh + sum_j p_j v_j and stores the new sum into fresh.
// SPLIT: workgroup x covers part x % nsplit of unit x / nsplit's list (its nsplit parts are equal runs of
// whole key blocks) and stores, per row, the unnormalised fp32 output of its part into out (rows of D
// floats, part-minor) and the part's running max and normaliser (base 2) as a float pair into lse; the
// merge kernel below combines the parts.
template <int D, int NW, bool DENSE, bool OUT_F32, bool DELTA, bool SPLIT>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(3, 3))) void attn_fwd_lean(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ counts, int cap,
    int Nq, int Nk, int group, int G, float scale_log2, void* __restrict__ out, float* __restrict__ lse,
    uint32_t n_units, const float* __restrict__ lse_in, const float* __restrict__ out_prev,
    float* __restrict__ fresh, int row0, int serial, int nsplit) {
  using L = FwdLayout<D, BKL>;
  constexpr int NRS = (L::ROWSETS + NW - 1) / NW;
  // The two stages' K and V tiles are separate LDS objects, so the compiler can tell that the reads of
  // one stage do not depend on the gather in flight into the other one (no wait for it).
  __shared__ __attribute__((aligned(1024))) char sk0[L::MAT_BYTES];
  __shared__ __attribute__((aligned(1024))) char sv0[L::MAT_BYTES];
  __shared__ __attribute__((aligned(1024))) char sk1[L::MAT_BYTES];
  __shared__ __attribute__((aligned(1024))) char sv1[L::MAT_BYTES];

  const uint32_t flat = xcd_striped(blockIdx.x, n_units, 128);
  const uint32_t unit = SPLIT ? flat / (uint32_t)nsplit : flat;
  const int part = SPLIT ? (int)(flat % (uint32_t)nsplit) : 0;
  const int g = (int)(unit % (uint32_t)G);
  const uint32_t bh = unit / (uint32_t)G;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hi = lane >> 5;
  const int ql = lane & 31;
  // this launch covers rows [row0, row0 + 32 NW) of the group (groups wider than 128 rows run as several
  // launches of at most four waves)
  const int r0 = g * group + row0;
  const int rows_here = min(min(group - row0, NW * 32), Nq - r0);
  if (rows_here <= 0) return;   // the partial last group may end before this launch's rows
  const int wrow = wave * 32 + ql;
  const bool row_valid = wrow < rows_here;

  int c;
  if (DENSE) {
    c = Nk;
  } else {
    c = counts[bh * (uint32_t)G + g];
    c = c < 0 ? 0 : (c > cap ? cap : c);
  }
  int lo = 0;   // this part's first list position
  if (SPLIT) {
    const int nb_all = (c + BKL - 1) / BKL;
    const int b0 = (int)((int64_t)part * nb_all / nsplit), b1 = (int)((int64_t)(part + 1) * nb_all / nsplit);
    lo = b0 * BKL;
    c = max(min(b1 * BKL, c) - lo, 0);
  }
  const int nblk = (c + BKL - 1) / BKL;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(k + (size_t)bh * Nk * D, (uint32_t)Nk * L::RB);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(v + (size_t)bh * Nk * D, (uint32_t)Nk * L::RB);
  const int32_t* ilist = DENSE ? nullptr : idx + ((size_t)bh * G + g) * (size_t)cap + lo;
  // the list through a buffer resource: 32-bit offsets, no 64-bit address arithmetic per load
  const __amdgpu_buffer_rsrc_t ri = make_rsrc(ilist, DENSE ? 0u : (uint32_t)c * 4u);

  bf16x8 qf[L::KSTEPS];
  {
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(q + (size_t)bh * Nq * D, (uint32_t)Nq * L::RB);
    const uint32_t rowoff = row_valid ? (uint32_t)(r0 + wrow) * L::RB : (uint32_t)Nq * L::RB;
#pragma unroll
    for (int ks = 0; ks < L::KSTEPS; ++ks)
      qf[ks] = __builtin_bit_cast(bf16x8, buffer_load_x4(rq, rowoff + (uint32_t)(2 * ks + hi) * 16));
  }
  uint32_t koff[L::KSTEPS];
#pragma unroll
  for (int ks = 0; ks < L::KSTEPS; ++ks) koff[ks] = ql * L::RB + 16 * ((2 * ks + hi) ^ L::swz_k(ql));
  const int s16 = lane & 15, g16 = lane >> 4;
  const int vrow = 4 * hi + (s16 >> 2);
  uint32_t voff[L::DBLK];
#pragma unroll
  for (int db = 0; db < L::DBLK; ++db)
    voff[db] = vrow * L::RB + 16 * ((4 * db + 2 * (g16 & 1) + ((s16 & 3) >> 1)) ^ L::swz_v(vrow)) + 8 * (s16 & 1);

  const int row_in = lane / L::NC;
  const int pchunk = lane % L::NC;
  uint32_t kch[NRS], vch[NRS];
#pragma unroll
  for (int j = 0; j < NRS; ++j) {
    const int row = (wave + j * NW) * L::ROWS_PER_LOAD + row_in;
    kch[j] = 16u * (uint32_t)(pchunk ^ L::swz_k(row));
    vch[j] = 16u * (uint32_t)(pchunk ^ L::swz_v(row));
  }
  int keys[NRS];
  auto fetch_keys = [&](int blk) {
#pragma unroll
    for (int j = 0; j < NRS; ++j) {
      const int rs = wave + j * NW;
      const int p = blk * BKL + rs * L::ROWS_PER_LOAD + row_in;
      if (DENSE) keys[j] = p < Nk ? p : Nk - 1;
      else if (L::ROWSETS % NW == 0 || rs < L::ROWSETS)
        keys[j] = __builtin_amdgcn_raw_buffer_load_b32(ri, (uint32_t)min(p, c - 1) * 4u, 0, 0);
    }
  };
  auto issue = [&](char* kst, char* vst) {
#pragma unroll
    for (int j = 0; j < NRS; ++j) {
      const int rs = wave + j * NW;
      if (L::ROWSETS % NW == 0 || rs < L::ROWSETS) {
        // an index outside [0, Nk) reads the zero row past the end of the buffer
        const uint32_t base = min((uint32_t)keys[j], (uint32_t)Nk) * L::RB;
        buffer_load_lds_x4(rk, kst + rs * L::ROWS_PER_LOAD * L::RB, base + kch[j]);
        buffer_load_lds_x4(rv, vst + rs * L::ROWS_PER_LOAD * L::RB, base + vch[j]);
      }
    }
  };

  f32x16 o[L::DBLK];
#pragma unroll
  for (int i = 0; i < L::DBLK; ++i) o[i] = f32x16{};
  float m_run = -INFINITY;
  if (DELTA) m_run = row_valid ? lse_in[(size_t)bh * Nq + r0 + wrow] * 1.4426950408889634f : 0.0f;
  // Row sums: v_mfma_f32_16x16x32_bf16 with A = the lane's 8 packed probabilities (row l % 16, k-group
  // l / 16) and B = this selector (column l % 16, k-group l / 16), which is one in column 0 for the even
  // k-groups (lanes l % 16 and 32 + l % 16, both query l % 16) and in column 1 for the odd ones (query
  // 16 + l % 16).  Lanes 16 g and 16 g + 1 then hold the sums of queries 4 g + i and 16 + 4 g + i in
  // lacc[i].  l_carry holds what was moved out of lacc when the running max moved (rare).
  const uint32_t selw = ((lane & 15) == ((lane >> 4) & 1)) ? 0x3F803F80u : 0u;
  const bf16x8 sel = __builtin_bit_cast(bf16x8, u32x4{selw, selw, selw, selw});
  f32x4 lacc = {};
  float l_carry = 0.0f;
  auto row_sum = [&]() {   // lacc's sum of this lane's query
    const int src = 16 * ((ql & 15) >> 2) + (ql >> 4);
    float t = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float li = lacc[i];   // (a bit cast of the vector element itself would read element 0)
      const float x = __int_as_float(__builtin_amdgcn_ds_bpermute(src * 4, __float_as_int(li)));
      if ((ql & 3) == i) t = x;
    }
    return t;
  };

  auto block = [&](auto st, auto first, int j) {
    constexpr int ST = decltype(st)::value;
    constexpr bool FIRST = decltype(first)::value != 0;   // block 0 sets the running max
    wait_vmcnt0();
    __syncthreads();
    if (j + 1 < nblk) {
      if (ST == 0) issue(sk1, sv1);
      else issue(sk0, sv0);
      if (j + 2 < nblk) fetch_keys(j + 2);
      if (serial) {   // pipeline depth 1: the next block's gather completes before this block computes
        wait_vmcnt0();
        __syncthreads();
      }
    }
    const char* sk = ST == 0 ? sk0 : sk1;
    const char* sv = ST == 0 ? sv0 : sv1;
    f32x16 sacc = {};
#pragma unroll
    for (int ks = 0; ks < L::KSTEPS; ++ks) {
      const bf16x8 a = *(const bf16x8*)(sk + koff[ks]);
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], sacc, 0, 0, 0);
    }
    if (j == nblk - 1 && (c & (BKL - 1))) {
      const int valid = c - j * BKL;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (8 * (r >> 2) + 4 * hi + (r & 3) >= valid) sacc[r] = -INFINITY;
    }
    // running max: taken on the first block; afterwards only when one of this block's probabilities
    // passes 2^64 (an exp overflow or a NaN does too)
    auto take_max = [&]() {
      float bmax = sacc[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) bmax = fmaxf(bmax, sacc[r]);
      bmax = pair_max(bmax) * scale_log2;
      const float mnew = fmaxf(m_run, bmax);
      const float alpha = (mnew == m_run) ? 1.0f : __builtin_amdgcn_exp2f(m_run - mnew);
      m_run = mnew;
      l_carry *= alpha;
#pragma unroll
      for (int i = 0; i < L::DBLK; ++i) o[i] *= alpha;
    };
    uint32_t pk[8];
    auto exps = [&]() {
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[r], scale_log2, -m_run));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[r + 1], scale_log2, -m_run));
        pk[r >> 1] = pack_bf16x2(p0, p1);
      }
    };
    if (!DELTA && FIRST) take_max();
    exps();
    if (!DELTA) {
      // largest probability of the lane, as bf16 bits, by packed 16-bit integer maxima
      u16x2 mx[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        mx[i] = __builtin_elementwise_max(__builtin_bit_cast(u16x2, pk[2 * i]), __builtin_bit_cast(u16x2, pk[2 * i + 1]));
      const u16x2 m2 = __builtin_elementwise_max(__builtin_elementwise_max(mx[0], mx[1]),
                                                 __builtin_elementwise_max(mx[2], mx[3]));
      const uint32_t top = m2[0] > m2[1] ? m2[0] : m2[1];
      if (__builtin_amdgcn_ballot_w64(top > RESCALE_BF16_BITS) != 0) {
        l_carry += row_sum();
        lacc = f32x4{};
        take_max();
        exps();
      }
    }
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const u32x4 bw = {pk[4 * tt], pk[4 * tt + 1], pk[4 * tt + 2], pk[4 * tt + 3]};
      if (!DELTA) lacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, bw), sel, lacc, 0, 0, 0);
#pragma unroll
      for (int db = 0; db < L::DBLK; ++db) {
        const char* p0 = sv + (tt * 16) * L::RB + voff[db];
        const i16x4 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(SATTN_LDS_PTR(i16x4, p0));
        const i16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(SATTN_LDS_PTR(i16x4, p0 + 8 * L::RB));
        const u32x2 w0 = __builtin_bit_cast(u32x2, t0);
        const u32x2 w1 = __builtin_bit_cast(u32x2, t1);
        const u32x4 aw = {w0[0], w0[1], w1[0], w1[1]};
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, aw), __builtin_bit_cast(bf16x8, bw),
                                                       o[db], 0, 0, 0);
      }
    }
  };

  if (nblk > 0) {
    fetch_keys(0);
    issue(sk0, sv0);
    if (nblk > 1) fetch_keys(1);
  }
  if (nblk > 0) block(IC<0>{}, IC<1>{}, 0);
  int j = 1;
  for (; j + 1 < nblk; j += 2) {
    block(IC<1>{}, IC<0>{}, j);
    block(IC<0>{}, IC<0>{}, j + 1);
  }
  if (j < nblk) block(IC<1>{}, IC<0>{}, j);

  if constexpr (DELTA) {
    if (row_valid) {
      const size_t orow = ((size_t)bh * Nq + r0 + wrow) * D;
#pragma unroll
      for (int db = 0; db < L::DBLK; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int d0 = 32 * db + 8 * i + 4 * hi;
          const f32x4 fo = *(const f32x4*)(fresh + orow + d0);
          const f32x4 op = *(const f32x4*)(out_prev + orow + d0);
          const f32x4 fn = {o[db][4 * i], o[db][4 * i + 1], o[db][4 * i + 2], o[db][4 * i + 3]};
          const f32x4 x = op - fo + fn;
          *(f32x4*)(fresh + orow + d0) = fn;
          if (OUT_F32) *(f32x4*)((float*)out + orow + d0) = x;
          else *(u32x2*)((uint16_t*)out + orow + d0) = u32x2{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
        }
    }
    return;
  }
  const float l_tot = l_carry + row_sum();
  if constexpr (SPLIT) {
    if (row_valid) {
      const size_t prow = ((size_t)bh * Nq + r0 + wrow) * (size_t)nsplit + part;
      float* po = (float*)out + prow * D;
#pragma unroll
      for (int db = 0; db < L::DBLK; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int d0 = 32 * db + 8 * i + 4 * hi;
          *(f32x4*)(po + d0) = f32x4{o[db][4 * i], o[db][4 * i + 1], o[db][4 * i + 2], o[db][4 * i + 3]};
        }
      if (hi == 0) *(f32x2*)(lse + 2 * prow) = f32x2{m_run, l_tot};
    }
    return;
  }
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  if (row_valid) {
    const size_t orow = ((size_t)bh * Nq + r0 + wrow) * D;
#pragma unroll
    for (int db = 0; db < L::DBLK; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d0 = 32 * db + 8 * i + 4 * hi;
        const float x0 = o[db][4 * i] * inv, x1 = o[db][4 * i + 1] * inv;
        const float x2 = o[db][4 * i + 2] * inv, x3 = o[db][4 * i + 3] * inv;
        if (OUT_F32) *(f32x4*)((float*)out + orow + d0) = f32x4{x0, x1, x2, x3};
        else *(u32x2*)((uint16_t*)out + orow + d0) = u32x2{pack_bf16x2(x0, x1), pack_bf16x2(x2, x3)};
      }
    if (lse != nullptr && hi == 0)
      lse[(size_t)bh * Nq + r0 + wrow] = l_tot > 0.0f ? (m_run + __log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
  }
}

template <int D, int NW, bool DENSE, bool DELTA>
static int launch_lean_t(const FwdArgs& a, int row0) {
  const uint32_t G = (uint32_t)((a.Nq + a.group - 1) / a.group);
  const uint32_t n_units = (uint32_t)a.B * (uint32_t)a.H * G;
  const float scale_log2 = a.scale * 1.4426950408889634f;
  hipStream_t st = (hipStream_t)a.stream;
  log_launch("attn_fwd_lean<D=%d, waves=%d, %s%s, %s> rows %d.. of each group: %u workgroups x %d threads%s", D, NW,
             DENSE ? "dense" : "sparse", DELTA ? " delta" : "", a.out_f32 ? "f32" : "bf16", row0, n_units, NW * 64,
             a.serial ? ", pipeline depth 1" : "");
  if (a.out_f32)
    hipLaunchKernelGGL((attn_fwd_lean<D, NW, DENSE, true, DELTA, false>), dim3(n_units), dim3(NW * 64), 0, st,
                       (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, a.idx, a.counts, a.cap,
                       a.Nq, a.Nk, a.group, (int)G, scale_log2, a.out, a.lse, n_units, a.lse_in, a.out_prev,
                       a.fresh, row0, a.serial ? 1 : 0, 1);
  else
    hipLaunchKernelGGL((attn_fwd_lean<D, NW, DENSE, false, DELTA, false>), dim3(n_units), dim3(NW * 64), 0, st,
                       (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, a.idx, a.counts, a.cap,
                       a.Nq, a.Nk, a.group, (int)G, scale_log2, a.out, a.lse, n_units, a.lse_in, a.out_prev,
                       a.fresh, row0, a.serial ? 1 : 0, 1);
  return (int)hipGetLastError();
}

// Groups of up to 128 rows: one launch, one wave per 32 rows.  Wider groups: the rows are cut into equal
// slices of at most 128 (192 -> 2 x 96, 256 -> 2 x 128), one launch per slice of every group.  A six- or
// eight-wave workgroup would gather each list once, but it places its waves two deep on some SIMDs and
// only one such workgroup then fits per CU at this kernel's register budget (1.4 waves per SIMD against
// 2.8).
template <int D, bool DELTA>
static int launch_sparse_d(const FwdArgs& a) {
  const int ns = (a.group + 127) / 128;
  const int slice = ((a.group + ns - 1) / ns + 31) / 32 * 32;
  for (int row0 = 0; row0 < a.group; row0 += slice) {
    const int waves = slice / 32;
    const int err = waves <= 2 ? launch_lean_t<D, 2, false, DELTA>(a, row0)
                  : waves == 3 ? launch_lean_t<D, 3, false, DELTA>(a, row0) : launch_lean_t<D, 4, false, DELTA>(a, row0);
    if (err) return err;
  }
  return 0;
}

template <int D>
static int launch_fwd_d(const FwdArgs& a) {
  if (a.dense) return launch_lean_t<D, 4, true, false>(a, 0);
  return a.delta ? launch_sparse_d<D, true>(a) : launch_sparse_d<D, false>(a);
}

int launch_attn_fwd(const FwdArgs& a) {
  return a.D == 64 ? launch_fwd_d<64>(a) : launch_fwd_d<128>(a);
}

// ---------------------------------------------------------------------------------------------
// Split lists: each unit's list in nsplit parts, one workgroup per part, then a merge
// ---------------------------------------------------------------------------------------------

// One wave per query row: out = sum_p w_p O_p / sum_p w_p l_p with w_p = 2^(m_p - max m) (a part with no
// keys has m_p = -inf and weight 0); lse = (max m + log2 sum_p w_p l_p) ln 2; a row with no keys at all
// gets out = 0 and lse = -inf, as in the single-pass forward.
template <int D, bool OUT_F32>
__global__ __launch_bounds__(256) void k_split_merge(const float* __restrict__ po, const f32x2* __restrict__ pml,
                                                     int nsplit, uint32_t rows, void* __restrict__ out,
                                                     float* __restrict__ lse) {
  constexpr int E = D / 64;   // dims per lane
  const uint32_t row = blockIdx.x * 4u + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  const f32x2* ml = pml + (size_t)row * nsplit;
  float m = -INFINITY;
  for (int p = 0; p < nsplit; ++p) m = fmaxf(m, ml[p][0]);
  float l = 0.0f, acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.0f;
  if (m > -INFINITY) {
    for (int p = 0; p < nsplit; ++p) {
      const f32x2 x = ml[p];
      if (x[0] == -INFINITY) continue;
      const float w = __builtin_amdgcn_exp2f(x[0] - m);
      l += w * x[1];
      const float* o = po + ((size_t)row * nsplit + p) * D + E * lane;
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] += w * o[e];
    }
  }
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  if (OUT_F32) {
#pragma unroll
    for (int e = 0; e < E; ++e) ((float*)out)[(size_t)row * D + E * lane + e] = acc[e] * inv;
  } else {
    if constexpr (E == 2) {
      ((uint32_t*)out)[((size_t)row * D + 2 * lane) / 2] = pack_bf16x2(acc[0] * inv, acc[1] * inv);
    } else {
      ((uint16_t*)out)[(size_t)row * D + lane] = (uint16_t)(pack_bf16x2(acc[0] * inv, 0.0f) & 0xffffu);
    }
  }
  if (lse != nullptr && lane == 0) lse[row] = l > 0.0f ? (m + __log2f(l)) * 0.69314718055994531f : -INFINITY;
}

template <int D, int NW>
static int launch_split_t(const FwdArgs& a, int row0, int nsplit, float* po, float* pml) {
  const uint32_t G = (uint32_t)((a.Nq + a.group - 1) / a.group);
  const uint32_t n_parts = (uint32_t)a.B * (uint32_t)a.H * G * (uint32_t)nsplit;
  const float scale_log2 = a.scale * 1.4426950408889634f;
  log_launch("attn_fwd_lean<D=%d, waves=%d, sparse, split in %d> rows %d.. of each group: %u workgroups x %d threads",
             D, NW, nsplit, row0, n_parts, NW * 64);
  hipLaunchKernelGGL((attn_fwd_lean<D, NW, false, false, false, true>), dim3(n_parts), dim3(NW * 64), 0,
                     (hipStream_t)a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, a.idx,
                     a.counts, a.cap, a.Nq, a.Nk, a.group, (int)G, scale_log2, (void*)po, pml, n_parts, nullptr,
                     nullptr, nullptr, row0, a.serial ? 1 : 0, nsplit);
  return (int)hipGetLastError();
}

template <int D>
static int launch_split_d(const FwdArgs& a, int nsplit, void* ws) {
  const size_t rows = (size_t)a.B * a.H * a.Nq;
  float* po = (float*)ws;
  float* pml = (float*)((char*)ws + split_partials_bytes(a.B, a.H, a.Nq, a.D, nsplit));
  // row slices of at most 128, as in launch_sparse_d
  const int ns = (a.group + 127) / 128;
  const int slice = ((a.group + ns - 1) / ns + 31) / 32 * 32;
  for (int row0 = 0; row0 < a.group; row0 += slice) {
    const int waves = slice / 32;
    const int err = waves <= 2 ? launch_split_t<D, 2>(a, row0, nsplit, po, pml)
                  : waves == 3 ? launch_split_t<D, 3>(a, row0, nsplit, po, pml)
                               : launch_split_t<D, 4>(a, row0, nsplit, po, pml);
    if (err) return err;
  }
  const dim3 grid((unsigned)((rows + 3) / 4));
  log_launch("k_split_merge<D=%d>: %zu rows of %d parts, %u workgroups x 256 threads", D, rows, nsplit, grid.x);
  if (a.out_f32)
    hipLaunchKernelGGL((k_split_merge<D, true>), grid, dim3(256), 0, (hipStream_t)a.stream, po, (const f32x2*)pml,
                       nsplit, (uint32_t)rows, a.out, a.lse);
  else
    hipLaunchKernelGGL((k_split_merge<D, false>), grid, dim3(256), 0, (hipStream_t)a.stream, po, (const f32x2*)pml,
                       nsplit, (uint32_t)rows, a.out, a.lse);
  return (int)hipGetLastError();
}

int launch_attn_fwd_split(const FwdArgs& a, int nsplit, void* ws) {
  return a.D == 64 ? launch_split_d<64>(a, nsplit, ws) : launch_split_d<128>(a, nsplit, ws);
}

}  // namespace sattn
