// Cached (full-attention) slice mask for gfx950.
//
// What is computed (FG-Attn review, Figure 10 and its list of free parameters): during a dense
// denoising iteration every M x 1 slice -- the M queries of a group against one key -- is marked
// when at least one of its full-attention softmax probabilities reaches tau (tau_cached = 0.5 / N
// on the pages).  With lse_i the row log-sum-exp that the dense forward already returns,
//
//     keep (g, j)  <=>  max over i in group g of  (scale q_i . k_j - lse_i)  >=  ln tau,
//
// and the kept keys of each group are emitted as an ascending index list with a count, the same
// structure the sparse forward consumes.
//
// Mapping onto CDNA4
// ------------------
//  * One workgroup per (batch, head, group); wave w owns query rows [32w, 32w+32).  The keys are
//    walked in contiguous blocks of 32, gathered into LDS with 16-byte buffer-load-to-LDS
//    instructions (double-buffered, rows past the end clamped to the last key).
//  * S = Q K^T with v_mfma_f32_32x32x16_bf16: A = the wave's 32 query rows (VGPRs, loaded once),
//    B = K rows from LDS.  In the accumulator layout a lane owns one key (lane % 32) and 16 query
//    rows, so the max over the group's queries is an in-lane max, one lane-pair exchange and an
//    OR over the waves.
//  * In base 2: x = s * scale * log2(e) - lse * log2(e), one FMA per score; rows outside the group
//    use lse = +inf and never pass.
//  * Each wave ballots "max x >= log2 tau" for the block's 32 keys and ORs the word into an LDS
//    bitmap of the group's keys; at the end the workgroup writes the ascending list from the
//    bitmap (popcounts, one block scan, then each thread emits the set bits of its words in order).
//
// The same walk also gives the column sums of Chipmunk's selection (Chipmunk review, Referee major
// comment 2: Alg. 4 ranks the columns of a chunk by their summed attention probabilities, with
// the normalisation constants of an earlier step): COLSUM = true sums exp2(x) over the group's
// rows instead of taking the max (in-lane sum, lane-pair sum, then the waves' partials in a fixed
// order) and stores the fp32 sums in the staging layout that the top-k selection reads.
#include <math.h>

#include <type_traits>

#include "../../include/sattn.h"
#include "device_common.hpp"
#include "launch.hpp"
#include "stage_layout.hpp"

namespace sattn {

namespace {

constexpr int CM_BK = 32;   // keys per block

template <int N>
using CmIC = std::integral_constant<int, N>;

template <int D>
struct CmLayout {
  static constexpr int RB = D * 2;                   // bytes per K row
  static constexpr int NC = D / 8;                   // 16-byte chunks per row
  static constexpr int ROWS_PER_LOAD = 1024 / RB;    // rows filled by one 64-lane 16-byte load
  static constexpr int ROWSETS = CM_BK / ROWS_PER_LOAD;
  static constexpr int STAGE_BYTES = CM_BK * RB;
  static constexpr int KSTEPS = D / 16;
  static constexpr int ROWDIV = 16 / NC;
  __device__ static inline int swz(int row) { return (row / ROWDIV) % NC; }
};

// Exclusive scan of one int per thread over a workgroup of NT threads; also returns the total.
template <int NT>
__device__ inline int wg_excl_scan(int x, int* wsum, int& total) {
  constexpr int NWV = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NWV; ++w) {
    const int s = wsum[w];
    before += (w < wave) ? s : 0;
    tot += s;
  }
  __syncthreads();
  total = tot;
  return before + incl - x;
}

}  // namespace

// Dynamic LDS: the group's key bitmap, ceil(Nk / 32) words (none for COLSUM).
template <int D, int NW, bool COLSUM>
__global__ __launch_bounds__(NW * 64) void k_cached_mask(const uint16_t* __restrict__ q,
                                                          const uint16_t* __restrict__ k,
                                                          const float* __restrict__ lse, int Nq, int Nk,
                                                          int group, int G, float scale_log2, float log2_tau,
                                                          int32_t* __restrict__ idx, int32_t* __restrict__ counts,
                                                          int cap, uint32_t n_units, float* __restrict__ csum,
                                                          float* __restrict__ csamp, int bh0) {
  using L = CmLayout<D>;
  constexpr int NT = NW * 64;
  constexpr int NRS = (L::ROWSETS + NW - 1) / NW;
  // The two stages are LDS objects of their own, so the compiler can tell that the reads of one stage
  // do not depend on the gather in flight into the other one (no wait for it).
  __shared__ __attribute__((aligned(1024))) char sk0[L::STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char sk1[L::STAGE_BYTES];
  __shared__ int wsum[NW];
  __shared__ float part[COLSUM ? 2 : 1][NW][32];
  extern __shared__ uint32_t bm[];

  const uint32_t unit = xcd_contiguous(blockIdx.x, n_units);
  const int g = (int)(unit % (uint32_t)G);
  const uint32_t bh = unit / (uint32_t)G + (uint32_t)bh0;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hi = lane >> 5, ql = lane & 31;
  const int r0 = g * group;
  const int rows_in_group = min(group, Nq - r0);
  const int nwords = (Nk + 31) / 32;
  const int nblk = nwords;

  if (!COLSUM)
    for (int w = tid; w < nwords; w += NT) bm[w] = 0u;
  // COLSUM: the column sums of block blk, summed over the waves in order, to the staging rows
  float* crow = COLSUM ? csum + (size_t)unit * score_stride(Nk) : nullptr;
  float* srow = COLSUM ? csamp + (size_t)unit * sample_stride(Nk) : nullptr;
  auto flush = [&](int blk) {
    if (wave == 0 && lane < 32) {
      const int key = blk * CM_BK + lane;
      float t = 0.0f;
#pragma unroll
      for (int w = 0; w < NW; ++w) t += part[blk & 1][w][lane];
      if (key < Nk) {
        crow[key] = t;
        if (key % SAMPLE_STEP == 0) srow[key / SAMPLE_STEP] = t;
      }
    }
  };

  // A operand: this lane's query row ql of the wave, chunk (2 ks + hi); rows outside the group read 0
  bf16x8 qf[L::KSTEPS];
  {
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(q + (size_t)bh * Nq * D, (uint32_t)Nq * L::RB);
    const int wrow = wave * 32 + ql;
    const uint32_t rowoff = wrow < rows_in_group ? (uint32_t)(r0 + wrow) * L::RB : (uint32_t)Nq * L::RB;
#pragma unroll
    for (int ks = 0; ks < L::KSTEPS; ++ks)
      qf[ks] = __builtin_bit_cast(bf16x8, buffer_load_x4(rq, rowoff + (uint32_t)(2 * ks + hi) * 16));
  }
  // lse (base 2) of the 16 query rows this lane holds in the accumulator: row 8(r/4) + 4 hi + r%4
  float lrow[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = wave * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
    lrow[r] = row < rows_in_group ? lse[(size_t)bh * Nq + r0 + row] * 1.4426950408889634f : INFINITY;
  }
  // B operand: K row ql of the block, chunk (2 ks + hi), XOR-swizzled in LDS
  uint32_t koff[L::KSTEPS];
#pragma unroll
  for (int ks = 0; ks < L::KSTEPS; ++ks) koff[ks] = ql * L::RB + 16 * ((2 * ks + hi) ^ L::swz(ql));

  const __amdgpu_buffer_rsrc_t rk = make_rsrc(k + (size_t)bh * Nk * D, (uint32_t)Nk * L::RB);
  const int row_in = lane / L::NC, pchunk = lane % L::NC;
  uint32_t kch[NRS];
#pragma unroll
  for (int j = 0; j < NRS; ++j) {
    const int row = (wave + j * NW) * L::ROWS_PER_LOAD + row_in;
    kch[j] = 16u * (uint32_t)(pchunk ^ L::swz(row));
  }
  auto issue = [&](char* st, int blk) {
#pragma unroll
    for (int j = 0; j < NRS; ++j) {
      const int rs = wave + j * NW;
      if (L::ROWSETS % NW == 0 || rs < L::ROWSETS) {
        const int p = blk * CM_BK + rs * L::ROWS_PER_LOAD + row_in;
        const uint32_t key = (uint32_t)(p < Nk ? p : Nk - 1);
        buffer_load_lds_x4(rk, st + rs * L::ROWS_PER_LOAD * L::RB, key * L::RB + kch[j]);
      }
    }
  };

  // block j reads stage j % 2 (even blocks stage 0)
  auto block = [&](auto stc, int j) {
    constexpr int st = decltype(stc)::value;
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt0();
    __syncthreads();   // stage j landed for every wave; stage j+1 is free again
    if (j + 1 < nblk) issue(st == 0 ? sk1 : sk0, j + 1);
    if (COLSUM && j > 0) flush(j - 1);   // every wave's partial of block j-1 is in LDS
    const char* sk = st == 0 ? sk0 : sk1;
    f32x16 acc = {};
#pragma unroll
    for (int ks = 0; ks < L::KSTEPS; ++ks) {
      const bf16x8 b = *(const bf16x8*)(sk + koff[ks]);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[ks], b, acc, 0, 0, 0);
    }
    if constexpr (COLSUM) {
      float ps = 0.0f;
#pragma unroll
      for (int r = 0; r < 16; ++r) ps += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[r], scale_log2, -lrow[r]));
      ps = pair_sum(ps);
      if (lane < 32) part[st][wave][lane] = ps;
    } else {
      float mx = __builtin_fmaf(acc[0], scale_log2, -lrow[0]);
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, __builtin_fmaf(acc[r], scale_log2, -lrow[r]));
      mx = pair_max(mx);
      const bool valid = j * CM_BK + ql < Nk;
      const uint64_t keep = __builtin_amdgcn_ballot_w64(valid && mx >= log2_tau);
      if (lane == 0 && (uint32_t)keep != 0u) atomicOr(&bm[j], (uint32_t)keep);
    }
  };
  issue(sk0, 0);
  int j = 0;
  for (; j + 1 < nblk; j += 2) {
    block(CmIC<0>{}, j);
    block(CmIC<1>{}, j + 1);
  }
  if (j < nblk) block(CmIC<0>{}, j);
  __syncthreads();
  if constexpr (COLSUM) {
    flush(nblk - 1);
    return;
  }

  // ascending list: each thread owns a contiguous run of words
  const int per = (nwords + NT - 1) / NT;
  const int w0 = min(tid * per, nwords), w1 = min(w0 + per, nwords);
  int mine = 0;
  for (int w = w0; w < w1; ++w) mine += __popc(bm[w]);
  int total;
  int pos = wg_excl_scan<NT>(mine, wsum, total);
  int32_t* out = idx + (size_t)unit * (size_t)cap;
  for (int w = w0; w < w1 && pos < cap; ++w) {
    uint32_t bits = bm[w];
    while (bits != 0u && pos < cap) {
      const int b = __builtin_ctz(bits);
      out[pos++] = w * 32 + b;
      bits &= bits - 1u;
    }
  }
  if (tid == 0) counts[unit] = min(total, cap);
}

template <int D, int NW>
static int launch_cached_t(const CachedMaskArgs& a) {
  const uint32_t G = (uint32_t)((a.Nq + a.group - 1) / a.group);
  const uint32_t n_units = (uint32_t)a.B * (uint32_t)a.H * G;
  const float scale_log2 = a.scale * 1.4426950408889634f;
  const float log2_tau = a.tau > 0.0f ? log2f(a.tau) : -INFINITY;
  const size_t lds = (size_t)((a.Nk + 31) / 32) * 4;   // at most 16 KB (Nk <= 131072)
  log_launch("k_cached_mask<D=%d, waves=%d>: %u workgroups x %d threads, %zu B of LDS bitmap", D, NW, n_units,
             NW * 64, lds);
  hipLaunchKernelGGL((k_cached_mask<D, NW, false>), dim3(n_units), dim3(NW * 64), lds, (hipStream_t)a.stream,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, a.lse, a.Nq, a.Nk, a.group, (int)G, scale_log2,
                     log2_tau, a.idx, a.counts, a.cap, n_units, nullptr, nullptr, 0);
  return (int)hipGetLastError();
}

template <int D>
static int launch_cached_d(const CachedMaskArgs& a) {
  const int waves = (a.group + 31) / 32;
  if (waves <= 2) return launch_cached_t<D, 2>(a);
  if (waves <= 4) return launch_cached_t<D, 4>(a);
  if (waves <= 6) return launch_cached_t<D, 6>(a);
  return launch_cached_t<D, 8>(a);
}

int launch_cached_mask(const CachedMaskArgs& a) {
  return a.D == 64 ? launch_cached_d<64>(a) : launch_cached_d<128>(a);
}

template <int D, int NW>
static int launch_colsum_t(const ColsumArgs& a) {
  const uint32_t G = (uint32_t)((a.Nq + a.group - 1) / a.group);
  const uint32_t n_units = (uint32_t)a.nheads * G;
  const float scale_log2 = a.scale * 1.4426950408889634f;
  log_launch("k_cached_mask<D=%d, waves=%d, column sums> heads %d..%d: %u workgroups x %d threads", D, NW, a.bh0,
             a.bh0 + a.nheads - 1, n_units, NW * 64);
  hipLaunchKernelGGL((k_cached_mask<D, NW, true>), dim3(n_units), dim3(NW * 64), 0, (hipStream_t)a.stream,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, a.lse, a.Nq, a.Nk, a.group, (int)G, scale_log2,
                     0.0f, nullptr, nullptr, 1, n_units, a.scores, a.samples, a.bh0);
  return (int)hipGetLastError();
}

template <int D>
static int launch_colsum_d(const ColsumArgs& a) {
  const int waves = (a.group + 31) / 32;
  if (waves <= 2) return launch_colsum_t<D, 2>(a);
  if (waves <= 4) return launch_colsum_t<D, 4>(a);
  if (waves <= 6) return launch_colsum_t<D, 6>(a);
  return launch_colsum_t<D, 8>(a);
}

int launch_colsum_scores(const ColsumArgs& a) {
  return a.D == 64 ? launch_colsum_d<64>(a) : launch_colsum_d<128>(a);
}

}  // namespace sattn
