// Refinement kernels for gfx950: exact scores of the candidates from their
// original int8 keys, the top-k of those, the hot-buffer resolve, and the
// gather of the misses from the full-history pool.
//
// Method: LeanSparse (arXiv 2611.04671), Abstract -- the original indexer
// keys are fetched only for the candidates the coarse pass kept.  Hot
// buffer: XM-Sparse digest, section on the hot buffer -- after the selection
// only the selected rows missing from the HBM hot buffer are fetched.
#include "ls_device.h"
#include "ls_select.h"
#include "ls_launch.h"
#include "ls_bucket.h"

namespace ls {

// ----------------------------------------------------- refine scores (A3) ---
//
// fs[b,c] = sum_h w[b,h] * max(0, q[b,h] . k8[b, cand[b,c]]).  16 candidates
// per tile feed v_mfma_i32_16x16x64_i8 directly: lane (n, g) gathers the
// 32-byte slice [32g, 32g+32) of candidate n's 128-byte key row (D = 128) or
// [16g, 16g+16) of its 64-byte row (D = 64); the query slice of the same
// dims is the A operand.  With a slot table it also stores each candidate's
// hot slot.  Per-head dots are exact in int32 (|dot| < 2^21);
// w * relu(dot) < 2^28 and groups of four stay below 2^30 before widening
// to int64.  Invalid candidates (-1) score 0 and are never selected.
// With a key cache, a candidate whose key row is resident in the request's
// cache is read from there, in HBM; the others from k8, which may then be
// pinned host memory read over PCIe.  KC = 1: residency from the slot table
// (kslot[t] in [0, key_slots)), one dependent load before the key load.
// KC = 2: from the commit's per-candidate code, loaded beside the candidate;
// a miss the commit gave a row (code -(2 + v)) is also copied into row v.
template <int D, int HT, int KC>
__global__ __launch_bounds__(256) void k_refine(const int8_t* __restrict__ q,
                                                const int8_t* __restrict__ w,
                                                const int8_t* __restrict__ k8,
                                                const int32_t* __restrict__ kslot,
                                                int8_t* __restrict__ kcache, int key_slots,
                                                const int32_t* __restrict__ kcode,
                                                const int32_t* __restrict__ cand,
                                                int64_t* __restrict__ fs,
                                                const int32_t* __restrict__ pos2slot,
                                                int32_t* __restrict__ cslot, int H, int max_ctx,
                                                int C) {
  constexpr int NMF = D / 64;
  const int b = blockIdx.y;
  const int l = lane_id(), n = l & 15, g = l >> 4;
  const int8_t* qb = q + (size_t)b * H * D;
  const int32_t* cb = cand + (size_t)b * C;

  const int c_base = blockIdx.x * kRefinePerWG + wave_id() * 64;
  const int8_t* kb = k8 + (size_t)b * max_ctx * D;
  const int32_t* ksb = KC == 1 ? kslot + (size_t)b * max_ctx : nullptr;
  const int32_t* kcd = KC == 2 ? kcode + (size_t)b * C : nullptr;
  int8_t* kcb = KC ? kcache + (size_t)b * key_slots * D : nullptr;
  int32_t code[4];
  // Every load below is unconditional (indices clamped, results selected
  // afterwards): a load under a divergent condition becomes a branch that
  // waits for it, which would serialise the whole prologue.
  // The candidate this lane reports, and its hot slot: looked up now, in
  // parallel with the key loads below.
  const int c_out = c_base + l;
  const int32_t p_raw = cb[min(c_out, C - 1)];
  const int32_t p_out = (c_out < C) ? p_raw : -1;
  int32_t pos[4];
  v4i raw[4][NMF];
#pragma unroll
  for (int tt = 0; tt < 4; tt++) {
    const int c = c_base + 16 * tt + n;
    const int32_t pr = cb[min(c, C - 1)];
    pos[tt] = (c < C) ? pr : -1;
    const int p = max(pos[tt], 0);
    const int8_t* row = kb + (size_t)p * D;
    if (KC == 1) {
      const int32_t ks = ksb[p];
      row = ((uint32_t)ks < (uint32_t)key_slots) ? kcb + (size_t)ks * D : row;
    }
    if (KC == 2) {
      const int32_t cr = kcd[min(c, C - 1)];
      code[tt] = (c < C && pos[tt] >= 0) ? cr : -1;
      row = ((uint32_t)code[tt] < (uint32_t)key_slots) ? kcb + (size_t)code[tt] * D : row;
    }
#pragma unroll
    for (int mf = 0; mf < NMF; mf++) {
      const int off = (D == 128) ? 32 * g + 16 * mf : 16 * g;
      raw[tt][mf] = *(const v4i*)(row + off);
    }
  }

  // hot slot of the reported candidate (without a table, a harmless read of
  // the candidate list stands in, so that no branch waits on the load)
  const int32_t* p2s = pos2slot ? pos2slot + (size_t)b * max_ctx : cb;
  const int32_t slot_raw = p2s[pos2slot ? max(p_out, 0) : 0];
  const int32_t slot_out = (p_out >= 0) ? slot_raw : 0;

  v4i qa[HT][NMF];
  int32_t wv[HT][4];
#pragma unroll
  for (int mt = 0; mt < HT; mt++) {
    const int h = 16 * mt + n;
#pragma unroll
    for (int mf = 0; mf < NMF; mf++) {
      const int off = (D == 128) ? 32 * g + 16 * mf : 16 * g;
      const v4i v = *(const v4i*)(qb + (size_t)min(h, H - 1) * D + off);
      qa[mt][mf] = (h < H) ? v : v4i{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int hh = 16 * mt + 4 * g + i;
      const int32_t wr = (int32_t)w[(size_t)b * H + min(hh, H - 1)];
      wv[mt][i] = hh < H ? wr : 0;
    }
  }

  int64_t part[4];
#pragma unroll
  for (int tt = 0; tt < 4; tt++) {
    v4i acc[HT];
#pragma unroll
    for (int mt = 0; mt < HT; mt++)
      acc[mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa[mt][0], raw[tt][0], v4i{0, 0, 0, 0}, 0,
                                                      0, 0);
    if (NMF == 2) {
#pragma unroll
      for (int mt = 0; mt < HT; mt++)
        acc[mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa[mt][NMF - 1], raw[tt][NMF - 1],
                                                        acc[mt], 0, 0, 0);
    }
    int64_t sum = 0;
#pragma unroll
    for (int mt = 0; mt < HT; mt++) {
      int32_t s4 = 0;
#pragma unroll
      for (int i = 0; i < 4; i++) s4 += wv[mt][i] * max(acc[mt][i], 0);
      sum += (int64_t)s4;
    }
    part[tt] = sum;
  }
  if (KC == 2) {
    // misses given a cache row: this lane's slices of the row it read
    // (stored after the MFMAs, so that no wait for the key loads comes
    // before the query loads)
#pragma unroll
    for (int tt = 0; tt < 4; tt++) {
      const int32_t v = -2 - code[tt];
      if (code[tt] <= -2 && v < key_slots) {
#pragma unroll
        for (int mf = 0; mf < NMF; mf++) {
          const int off = (D == 128) ? 32 * g + 16 * mf : 16 * g;
          *(v4i*)(kcb + (size_t)v * D + off) = raw[tt][mf];
        }
      }
    }
  }

  // reduce-scatter over the four lane groups: lane (n, g) ends with tile g
  const int64_t score = (int64_t)reduce_scatter4((uint64_t)part[0], (uint64_t)part[1],
                                                 (uint64_t)part[2], (uint64_t)part[3]);
  if (c_out < C) {
    fs[(size_t)b * C + c_out] = (p_out >= 0) ? score : 0;
    // the candidate's hot slot, looked up here where the lookups spread over
    // the whole grid, for the per-request top-k to read coalesced
    if (pos2slot) cslot[(size_t)b * C + c_out] = slot_out;
  }
}

// ---------------------------------------------- top-k + resolve (A4, A5) ----
//
// 1024-thread workgroups (k_topk_hist: one per 1024-candidate slice of a
// request; k_topk: one per request) keep min(K, valid) candidates under
// (fine score desc, position asc) and emit them in candidate order, i.e.
// ascending position.  With a slot table the emission also resolves each
// kept token against the hot buffer: rows[j] = its slot if resident, else
// hot_slots + (its rank among the misses); the misses' positions go to
// miss_pos in the same order.
//
// k_topk_hist (C <= 16384): thread t holds candidates t, t + 1024, ... in
// registers (coalesced loads).  Their fine scores are bucketed (float-like,
// 6 mantissa bits, both signs) into an LDS histogram; one scan from the top
// finds the bucket beta where the count crosses K.  Candidates above beta
// are kept; the few in beta go to an LDS tie list that one wave resolves
// exactly with the radix threshold search.  Output offsets come from wave
// ballots plus one small table of per-wave counts that wave 0 scans, so the
// kept candidates are written by consecutive lanes to consecutive slots.
// The candidates' hot slots were looked up by the refine kernel.
// A request runs PER workgroups (grid.x): every one makes the whole
// selection (the candidates are 16 B each, read from L2), then writes only
// its slice of 1024 candidates (k = its index) at the offsets the shared scan
// gives.
//
// k_topk (any C, also the fallback when the tie list overflows LDS): the
// block radix threshold search over all candidates.
constexpr int kTopkThreads = 1024;
constexpr int kTopkLds = 8192;
constexpr int kFineBinsPad = 8192;  // wide buckets, padded to 8 per thread
constexpr int kTopkTieLds = 8192;

template <int PER>
__global__ __launch_bounds__(kTopkThreads) void k_topk_hist(
    const int32_t* __restrict__ cand, const int64_t* __restrict__ fs,
    const int32_t* __restrict__ cslot, int32_t* __restrict__ topk,
    int64_t* __restrict__ topk_score, const int32_t* __restrict__ pos2slot,
    int32_t* __restrict__ rows, int32_t* __restrict__ n_miss, int32_t* __restrict__ miss_pos,
    int32_t* __restrict__ srcw, int hot_slots, int max_ctx, int C, int K) {
  constexpr int NT = kTopkThreads;
  constexpr int NW = NT / kWave;
  constexpr int BPT = kFineBinsPad / NT;  // bins per thread
  constexpr int NTAB = PER * NW;          // per-(k, wave) count table
  __shared__ uint32_t scan_sh[NW];
  __shared__ SelectShared ssh;
  __shared__ __attribute__((aligned(16))) uint32_t hist[kFineBinsPad];
  __shared__ int64_t tie_f[kTopkTieLds];
  __shared__ int32_t tie_c[kTopkTieLds];
  __shared__ uint32_t tab[NTAB];
  __shared__ uint32_t ttab[NTAB];  // ties per (batch, wave), for ranks by position
  __shared__ Threshold sh_thr;
  __shared__ ThresholdScratch thr_sc;  // the tie search's short list
  __shared__ int sh_beta;
  __shared__ uint32_t sh_above, n_tie;
  // (slice, request), numbered so that a request's workgroups share an XCD's
  // L2 (they all read the request's candidates)
  const int lin = xcd_major(blockIdx.x + gridDim.x * blockIdx.y, gridDim.x * gridDim.y);
  const int m = lin % gridDim.x, b = lin / gridDim.x;
  const int tid = threadIdx.x, l = lane_id(), wv = wave_id();
  const int32_t* cb = cand + (size_t)b * C;
  const int64_t* fb = fs + (size_t)b * C;

  int32_t c[PER];
  int64_t f[PER];
  // unconditional loads (clamped index, result selected afterwards)
  const bool resolve = pos2slot != nullptr;
  const int32_t* csb = cslot + (size_t)b * C;
  int32_t slot[PER];
#pragma unroll
  for (int k = 0; k < PER; k++) {
    const int i = tid + NT * k;
    const int ic = min(i, C - 1);
    const int32_t cr = cb[ic];
    const int64_t fr = fb[ic];
    const int32_t sr = csb[ic];  // hot slots of the candidates (refine kernel)
    const bool in = i < C;
    c[k] = in ? cr : -1;
    f[k] = in ? fr : 0;
    slot[k] = (resolve && in) ? sr : 0;
  }
#pragma unroll
  for (int k = 0; k < BPT; k++) hist[tid * BPT + k] = 0;
  if (tid == 0) {
    sh_beta = -1;
    sh_above = 0;
    n_tie = 0;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < PER; k++)
    if (c[k] >= 0) atomicAdd(&hist[wide_bucket(f[k])], 1u);
  __syncthreads();

  // bucket where the count from the top crosses K (thread 0: top bins)
  const int seg = NT - 1 - tid;
  uint32_t hc[BPT];
  uint32_t s = 0;
#pragma unroll
  for (int k = 0; k < BPT; k++) {
    hc[k] = hist[seg * BPT + k];
    s += hc[k];
  }
  uint32_t n_c;
  const uint32_t above_seg = block_excl_scan<NT>(s, scan_sh, &n_c);
  const uint32_t need_all = min((uint32_t)K, n_c);
  if (need_all < n_c && above_seg < need_all && need_all <= above_seg + s) {
    uint32_t run = above_seg;
#pragma unroll
    for (int k = BPT - 1; k >= 0; k--) {
      if (run < need_all && run + hc[k] >= need_all) {
        sh_beta = seg * BPT + k;
        sh_above = run;
      }
      run += hc[k];
    }
  }
  __syncthreads();
  const int beta = sh_beta;  // -1: every valid candidate is kept

  bool sel[PER];
  if (beta < 0) {
#pragma unroll
    for (int k = 0; k < PER; k++) sel[k] = c[k] >= 0;
  } else {
    const uint32_t need = need_all - sh_above;  // 1 <= need <= ties
    // bucket beta holds the scores [b_lo, b_hi] (buckets are contiguous
    // ranges, so comparing a score with them places it as its bucket would,
    // without keeping the buckets in registers)
    int64_t b_lo, b_hi;
    wide_bucket_range(beta, b_lo, b_hi);
    // the wave's ties of all PER batches, with one reservation in the list
    uint64_t mt[PER];
    uint32_t wave_ties = 0;
#pragma unroll
    for (int k = 0; k < PER; k++) {
      mt[k] = __ballot(c[k] >= 0 && f[k] >= b_lo && f[k] <= b_hi);
      wave_ties += (uint32_t)__popcll(mt[k]);
    }
    if (wave_ties) {  // wave-uniform
      uint32_t base = 0;
      if (l == 0) base = atomicAdd(&n_tie, wave_ties);
      uint32_t i = wave_read(base, 0);
#pragma unroll
      for (int k = 0; k < PER; k++) {
        const bool tie = (mt[k] >> l) & 1ull;
        const uint32_t j = i + lane_rank(mt[k]);
        if (tie && j < (uint32_t)kTopkTieLds) {
          tie_f[j] = f[k];
          tie_c[j] = c[k];
        }
        i += (uint32_t)__popcll(mt[k]);
      }
    }
    __syncthreads();
    const uint32_t nt = n_tie;
    const bool overflow = nt > (uint32_t)kTopkTieLds;
    Threshold thr{0ull, 0u, 0};
    // A long tie list may be one run of equal scores (repeated content, or the
    // identical planted tokens of the synthetic workloads): then the cut is the
    // need-th tie in position order, found without searching the list.  Only
    // long lists are checked, so the common path pays one uniform branch.
    bool one_key = false;
    if (need < nt && nt > (uint32_t)kWaveTies) {  // workgroup-uniform
      const int64_t ref = tie_f[0];  // the first reserved entry (nt >= 1)
      bool same = true;
#pragma unroll
      for (int k = 0; k < PER; k++) same = same && !(((mt[k] >> l) & 1ull) && f[k] != ref);
      if (l == 0) {
#pragma unroll
        for (int k = 0; k < PER; k++) ttab[k * NW + wv] = (uint32_t)__popcll(mt[k]);
      }
      one_key = __syncthreads_and(same) != 0;
    }
    if (one_key) {  // workgroup-uniform
      // Every tie has the same key (a group of equal scores at the cut): the
      // cut is the need-th tie in position order, and the candidates are in
      // position order (index k * NT + tid), so a tie's rank is the ties
      // before its (batch, wave) entry plus its rank in the wave's ballot --
      // no search over the list.  Each wave scans the count table itself.
      constexpr int Q = NTAB >= kWave ? NTAB / kWave : 1;
      uint32_t v[Q];
      uint32_t sum = 0;
#pragma unroll
      for (int q = 0; q < Q; q++) {
        const int e = l * Q + q;
        v[q] = e < NTAB ? ttab[e] : 0u;
        sum += v[q];
      }
      const uint32_t excl = wave_incl_scan(sum) - sum;
#pragma unroll
      for (int k = 0; k < PER; k++) {
        const int e = k * NW + wv;  // entry (k, wave): lane e / Q, position e % Q
        uint32_t run = excl;
#pragma unroll
        for (int q = 0; q < Q; q++)
          if (q < e % Q) run += v[q];
        const uint32_t pre = wave_read(run, e / Q);
        if (((mt[k] >> l) & 1ull) && pre + lane_rank(mt[k]) == need - 1u)
          sh_thr = Threshold{key_of_i64(f[k]), (uint32_t)c[k], 1};
      }
      __syncthreads();
      thr = sh_thr;
    } else if (overflow) {  // every valid candidate takes part: the cut is exact on its own
      auto get = [&](int i, uint64_t& u, uint32_t& p) {
        u = key_of_i64(fb[i]);
        p = (uint32_t)cb[i];
      };
      thr = block_threshold<NT>(get, (int)n_c, need_all, ssh);
    } else if (need < nt) {
      auto get = [&](int i, uint64_t& u, uint32_t& p) {
        u = key_of_i64(tie_f[i]);
        p = (uint32_t)tie_c[i];
      };
      thr = tie_threshold<NT>(get, (int)nt, need, ssh, &thr_sc, &sh_thr, key_of_i64(b_lo),
                              key_of_i64(b_hi), pos_bits_below(max_ctx));
    }
#pragma unroll
    for (int k = 0; k < PER; k++) {
      const bool v = c[k] >= 0;
      if (overflow)
        sel[k] = v && keep(thr, key_of_i64(f[k]), (uint32_t)c[k]);
      else
        sel[k] = v && (f[k] > b_hi ||
                       (f[k] >= b_lo && keep(thr, key_of_i64(f[k]), (uint32_t)c[k])));
    }
  }

  // ---- emission in candidate order
  uint64_t ms[PER], mm[PER];
#pragma unroll
  for (int k = 0; k < PER; k++) {
    ms[k] = __ballot(sel[k]);
    mm[k] = __ballot(sel[k] && slot[k] < 0);
    // kept and missed counts, packed (both stay below 2^16)
    if (l == 0) tab[k * NW + wv] = (uint32_t)__popcll(ms[k]) | ((uint32_t)__popcll(mm[k]) << 16);
  }
  __syncthreads();
  // every wave scans the table itself (exclusive, in (k, wave) order) and
  // keeps the offset of its own entry of slice m: no second barrier
  uint32_t my_base, tot;
  {
    constexpr int Q = NTAB >= kWave ? NTAB / kWave : 1;
    uint32_t v[Q];
    uint32_t sum = 0;
#pragma unroll
    for (int q = 0; q < Q; q++) {
      const int e = l * Q + q;
      v[q] = e < NTAB ? tab[e] : 0u;
      sum += v[q];
    }
    const uint32_t incl = wave_incl_scan(sum);
    tot = wave_read(incl, kWave - 1);
    // entry (m, wv) sits at e = m * NW + wv: lane e / Q, position e % Q
    const int e_me = m * NW + wv;
    uint32_t run = incl - sum;
#pragma unroll
    for (int q = 0; q < Q; q++)
      if (q < e_me % Q) run += v[q];
    my_base = wave_read(run, e_me / Q);
  }
  int32_t* tb = topk + (size_t)b * K;
  int64_t* sb = topk_score ? topk_score + (size_t)b * K : nullptr;
  int32_t* rb = rows ? rows + (size_t)b * K : nullptr;
  int32_t* mb = miss_pos ? miss_pos + (size_t)b * K : nullptr;
  int32_t* xb = srcw ? srcw + (size_t)b * K : nullptr;
#pragma unroll
  for (int k = 0; k < PER; k++) {
    if (k != m) continue;  // this workgroup's slice (workgroup-uniform)
    const uint32_t base = my_base;
    const uint32_t o = (base & 0xFFFFu) + lane_rank(ms[k]);
    if (!sel[k] || o >= (uint32_t)K) continue;  // exactly min(K, valid) are kept
    tb[o] = c[k];
    if (sb) sb[o] = f[k];
    if (resolve) {
      if (slot[k] >= 0) {
        rb[o] = slot[k];
      } else {
        const uint32_t om = (base >> 16) + lane_rank(mm[k]);
        rb[o] = hot_slots + (int32_t)om;
        mb[om] = c[k];
      }
      // the pool position of a miss (for a gathering attention), -1 for a hit
      if (xb) xb[o] = slot[k] >= 0 ? -1 : c[k];
    }
  }
  if (m == 0) {
    for (int j = (int)(tot & 0xFFFFu) + tid; j < K; j += NT) {
      tb[j] = -1;
      if (sb) sb[j] = 0;
      if (rb) rb[j] = -1;
      if (xb) xb[j] = -1;
    }
    if (tid == 0 && n_miss) n_miss[b] = resolve ? (int32_t)(tot >> 16) : 0;
  }
}

__global__ __launch_bounds__(kTopkThreads) void k_topk(
    const int32_t* __restrict__ cand, const int64_t* __restrict__ fs, int32_t* __restrict__ topk,
    int64_t* __restrict__ topk_score, const int32_t* __restrict__ pos2slot,
    int32_t* __restrict__ rows, int32_t* __restrict__ n_miss, int32_t* __restrict__ miss_pos,
    int32_t* __restrict__ srcw, int hot_slots, int max_ctx, int C, int K) {
  constexpr int NT = kTopkThreads;
  __shared__ uint32_t scan_sh[NT / kWave];
  __shared__ SelectShared ssh;
  __shared__ int64_t lds_f[kTopkLds];
  __shared__ int32_t lds_c[kTopkLds];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int32_t* cb = cand + (size_t)b * C;
  const int64_t* fb = fs + (size_t)b * C;

  // valid candidates form a prefix (ascending, -1 padded)
  uint32_t nv = 0;
  for (int i = tid; i < C; i += NT) nv += (cb[i] >= 0) ? 1u : 0u;
  uint32_t n_c;
  block_excl_scan<NT>(nv, scan_sh, &n_c);
  const bool in_lds = n_c <= (uint32_t)kTopkLds;
  if (in_lds) {
    for (int i = tid; i < (int)n_c; i += NT) {
      lds_f[i] = fb[i];
      lds_c[i] = cb[i];
    }
    __syncthreads();
  }
  const int64_t* ff = in_lds ? lds_f : fb;
  const int32_t* cc = in_lds ? lds_c : cb;

  const uint32_t need = min((uint32_t)K, n_c);
  const bool all = need >= n_c;
  Threshold thr{0ull, 0u, 0};
  if (!all) {
    auto get = [&](int i, uint64_t& u, uint32_t& p) {
      u = key_of_i64(ff[i]);
      p = (uint32_t)cc[i];
    };
    thr = block_threshold<NT>(get, (int)n_c, need, ssh);
  }

  const int32_t* p2s = pos2slot ? pos2slot + (size_t)b * max_ctx : nullptr;
  const int per = ((int)n_c + NT - 1) / NT;
  const int i0 = tid * per, i1 = min(i0 + per, (int)n_c);
  uint32_t c_sel = 0, c_miss = 0;
  for (int i = i0; i < i1; i++) {
    const bool s = all || keep(thr, key_of_i64(ff[i]), (uint32_t)cc[i]);
    if (s) {
      c_sel++;
      if (p2s && p2s[cc[i]] < 0) c_miss++;
    }
  }
  uint32_t tot_sel, tot_miss;
  uint32_t o_sel = block_excl_scan<NT>(c_sel, scan_sh, &tot_sel);
  uint32_t o_miss = block_excl_scan<NT>(c_miss, scan_sh, &tot_miss);
  int32_t* tb = topk + (size_t)b * K;
  int64_t* sb = topk_score ? topk_score + (size_t)b * K : nullptr;
  int32_t* rb = rows ? rows + (size_t)b * K : nullptr;
  int32_t* mb = miss_pos ? miss_pos + (size_t)b * K : nullptr;
  int32_t* xb = srcw ? srcw + (size_t)b * K : nullptr;
  for (int i = i0; i < i1; i++) {
    const int32_t p = cc[i];
    if (!(all || keep(thr, key_of_i64(ff[i]), (uint32_t)p))) continue;
    if (o_sel < (uint32_t)K) {
      tb[o_sel] = p;
      if (sb) sb[o_sel] = ff[i];
      if (p2s) {
        const int32_t slot = p2s[p];
        if (slot >= 0) {
          rb[o_sel] = slot;
        } else {
          rb[o_sel] = hot_slots + (int32_t)o_miss;
          mb[o_miss] = p;
          o_miss++;
        }
        if (xb) xb[o_sel] = slot >= 0 ? -1 : p;
      }
    }
    o_sel++;
  }
  for (int j = (int)tot_sel + tid; j < K; j += NT) {
    tb[j] = -1;
    if (sb) sb[j] = 0;
    if (rb) rb[j] = -1;
    if (xb) xb[j] = -1;
  }
  if (tid == 0 && n_miss) n_miss[b] = p2s ? (int32_t)tot_miss : 0;
}

hipError_t launch_refine_topk(const int8_t* q, const int8_t* w, const KeySource& keys,
                              const int32_t* cand, const RefineWS& ws, int32_t* topk,
                              int64_t* topk_score, const int32_t* pos2slot, int32_t* rows,
                              int32_t* n_miss, int hot_slots, int B, int H, int D, int max_ctx,
                              int C, int K, hipStream_t st) {
  dim3 grid((C + kRefinePerWG - 1) / kRefinePerWG, B);
  const int HT = (H + 15) / 16;
#define LS_REFINE_KC(DD, TT, KC)                                                             \
  hipLaunchKernelGGL((k_refine<DD, TT, KC>), grid, dim3(256), 0, st, q, w, keys.k8, keys.kslot, \
                     keys.kcache, keys.key_slots, keys.code, cand, ws.fs, pos2slot, ws.slot, H, \
                     max_ctx, C)
#define LS_REFINE(DD, TT)                                                                     \
  do {                                                                                        \
    if (keys.key_slots > 0 && keys.code) LS_REFINE_KC(DD, TT, 2);                             \
    else if (keys.key_slots > 0) LS_REFINE_KC(DD, TT, 1);                                     \
    else LS_REFINE_KC(DD, TT, 0);                                                             \
  } while (0)
  if (D == 128) {
    if (HT == 1) LS_REFINE(128, 1); else if (HT == 2) LS_REFINE(128, 2);
    else if (HT == 3) LS_REFINE(128, 3); else LS_REFINE(128, 4);
  } else {
    if (HT == 1) LS_REFINE(64, 1); else if (HT == 2) LS_REFINE(64, 2);
    else if (HT == 3) LS_REFINE(64, 3); else LS_REFINE(64, 4);
  }
#undef LS_REFINE
#undef LS_REFINE_KC
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  int32_t* srcw = pos2slot ? ws.src : nullptr;
#define LS_TOPK(P)                                                                           \
  hipLaunchKernelGGL(k_topk_hist<P>, dim3(P, B), dim3(kTopkThreads), 0, st, cand, ws.fs,       \
                     ws.slot, topk, topk_score, pos2slot, rows, n_miss, ws.miss_pos, srcw,     \
                     hot_slots, max_ctx, C, K)
  if (C <= kTopkThreads) LS_TOPK(1);
  else if (C <= 2 * kTopkThreads) LS_TOPK(2);
  else if (C <= 4 * kTopkThreads) LS_TOPK(4);
  else if (C <= 8 * kTopkThreads) LS_TOPK(8);
  else if (C <= 16 * kTopkThreads) LS_TOPK(16);
  else
    hipLaunchKernelGGL(k_topk, dim3(B), dim3(kTopkThreads), 0, st, cand, ws.fs, topk, topk_score,
                       pos2slot, rows, n_miss, ws.miss_pos, srcw, hot_slots, max_ctx, C, K);
#undef LS_TOPK
  return hipGetLastError();
}

// ------------------------------------------------------ hot resolve (A5) ----
// Standalone resolve of an existing selection (one workgroup per request):
// the selection is ascending and -1 padded.
__global__ __launch_bounds__(256) void k_hot_resolve(const int32_t* __restrict__ topk,
                                                     const int32_t* __restrict__ pos2slot,
                                                     int32_t* __restrict__ rows,
                                                     int32_t* __restrict__ n_miss,
                                                     int32_t* __restrict__ miss_pos,
                                                     int hot_slots, int max_ctx, int K) {
  __shared__ uint32_t scan_sh[4];
  const int b = blockIdx.x;
  const int32_t* tb = topk + (size_t)b * K;
  uint32_t nv = 0;
  for (int i = threadIdx.x; i < K; i += 256) nv += (tb[i] >= 0) ? 1u : 0u;
  uint32_t n_sel;
  block_excl_scan<256>(nv, scan_sh, &n_sel);
  const int32_t* p2s = pos2slot + (size_t)b * max_ctx;
  const int per = (K + 255) / 256;
  const int i0 = threadIdx.x * per, i1 = min(i0 + per, (int)n_sel);
  uint32_t c_miss = 0;
  for (int i = i0; i < i1; i++) c_miss += (p2s[tb[i]] < 0) ? 1u : 0u;
  uint32_t tot;
  uint32_t o = block_excl_scan<256>(c_miss, scan_sh, &tot);
  int32_t* rb = rows + (size_t)b * K;
  int32_t* mb = miss_pos + (size_t)b * K;
  for (int i = i0; i < i1; i++) {
    const int32_t p = tb[i];
    const int32_t slot = p2s[p];
    if (slot >= 0) {
      rb[i] = slot;
    } else {
      rb[i] = hot_slots + (int32_t)o;
      mb[o] = p;
      o++;
    }
  }
  for (int i = (int)n_sel + threadIdx.x; i < K; i += 256) rb[i] = -1;
  if (threadIdx.x == 0) n_miss[b] = (int32_t)tot;
}

hipError_t launch_hot_resolve(const int32_t* topk, const int32_t* pos2slot, int32_t* rows,
                              int32_t* n_miss, int32_t* miss_pos, int hot_slots, int B,
                              int max_ctx, int K, hipStream_t st) {
  hipLaunchKernelGGL(k_hot_resolve, dim3(B), dim3(256), 0, st, topk, pos2slot, rows, n_miss,
                     miss_pos, hot_slots, max_ctx, K);
  return hipGetLastError();
}

// ------------------------------------------------------- miss gather (A6) ---
// hot[b, hot_slots + j] := pool[b, miss_pos[b, j]] for j < n_miss[b], in
// 16-byte pieces: each workgroup copies a contiguous share of the request's
// pieces, every thread four pieces at a time with all loads issued before
// the stores.  The pool may be pinned host memory (reads then cross PCIe).

constexpr int kGatherWGPerReq = 32;
constexpr int kGatherUnroll = 4;

//
// With DST (a hot-buffer commit ran), miss j goes to the slot miss_dst[j]
// when it has one, else to scratch row hot_slots + j; the stores then go
// through a resource over the request's whole buffer, and pieces past the
// miss count get an offset beyond it.
//
// HOST (the pool is pinned host memory): the miss count is waited for before
// any row load, and pieces past it are not loaded at all -- a speculative
// load would be a wasted PCIe read there.
template <bool DST, bool HOST>
__global__ __launch_bounds__(256) void k_hot_gather(const int32_t* __restrict__ miss_pos,
                                                    const int32_t* __restrict__ n_miss,
                                                    const int32_t* __restrict__ miss_dst,
                                                    const uint4* pool, uint4* __restrict__ hot,
                                                    int hot_slots, int max_ctx, int K,
                                                    int chunks) {
  // Workgroup x copies misses x, x + G, x + 2G, ... (G workgroups per
  // request), as 16-byte pieces numbered (slot m of its list, chunk c) in
  // order, kGatherUnroll pieces per thread per round.  Positions and rows
  // load speculatively -- indices clamped, so every access stays inside the
  // lists and the pool -- at the same time as the miss count.  The stores go
  // through a buffer resource over the n_miss rows of the list: pieces of
  // slots past the count are dropped by the hardware, with no branch (a
  // branch would let the compiler sink each row load into it).
  const int b = blockIdx.y;
  const int G = gridDim.x;
  const int32_t* mp = miss_pos + (size_t)b * K;
  const uint4* pb = pool + (size_t)b * max_ctx * chunks;
  uint4* hb = hot + ((size_t)b * (hot_slots + K) + (DST ? 0 : hot_slots)) * chunks;
  const int32_t* md = DST ? miss_dst + (size_t)b * K : nullptr;
  const uint32_t whole = (uint32_t)(hot_slots + K) * (uint32_t)chunks * 16u;
  const int nm_raw = n_miss[b];
  // one round of kGatherUnroll pieces per thread from piece f0 on: every
  // position, then every row, then (after the fence) the stores
  auto round = [&](uint32_t f0, int nm) {
    uint4 v[kGatherUnroll];
    uint32_t off[kGatherUnroll], c[kGatherUnroll];
    int32_t p[kGatherUnroll], d[kGatherUnroll], j[kGatherUnroll];
#pragma unroll
    for (int u = 0; u < kGatherUnroll; u++) {
      const uint32_t f = f0 + threadIdx.x + 256u * u;
      const uint32_t m = f / (uint32_t)chunks;
      c[u] = f - m * (uint32_t)chunks;
      const int jj = blockIdx.x + G * (int)m;
      j[u] = jj;
      off[u] = ((uint32_t)jj * (uint32_t)chunks + c[u]) * 16u;
      p[u] = mp[min(jj, K - 1)];
      if (DST) d[u] = md[min(jj, K - 1)];
    }
    if (HOST && nm < 0) nm = min(max(nm_raw, 0), K);
#pragma unroll
    for (int u = 0; u < kGatherUnroll; u++) {
      const size_t src = (size_t)min(max(p[u], 0), max_ctx - 1) * chunks + c[u];
      if (HOST)
        v[u] = j[u] < nm ? pb[src] : uint4{0, 0, 0, 0};
      else
        v[u] = pb[src];
    }
    __builtin_amdgcn_sched_barrier(0);
    if (nm < 0) nm = min(max(nm_raw, 0), K);  // a list never holds more than K misses
    if (DST) {
#pragma unroll
      for (int u = 0; u < kGatherUnroll; u++) {
        const int32_t row = (d[u] >= 0 && d[u] < hot_slots) ? d[u] : hot_slots + j[u];
        off[u] = j[u] < nm ? ((uint32_t)row * (uint32_t)chunks + c[u]) * 16u : whole;
      }
    }
    const __amdgpu_buffer_rsrc_t hres =
        buffer_rsrc(hb, DST ? whole : (uint32_t)nm * (uint32_t)chunks * 16u);
#pragma unroll
    for (int u = 0; u < kGatherUnroll; u++)
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i, v[u]), hres, off[u], 0, 0);
    return nm;
  };
  constexpr uint32_t kRound = 256u * kGatherUnroll;
  const int nm = round(0u, -1);
  // slots of this workgroup (uniform); more rounds only past the first
  // kRound pieces
  const uint32_t my = nm > (int)blockIdx.x ? (uint32_t)((nm - 1 - (int)blockIdx.x) / G + 1) : 0u;
  for (uint32_t f0 = kRound; f0 < my * (uint32_t)chunks; f0 += kRound) round(f0, nm);
}

hipError_t launch_hot_gather(const int32_t* miss_pos, const int32_t* n_miss,
                             const int32_t* miss_dst, const void* pool, void* hot, int hot_slots,
                             int B, int max_ctx, int K, int row_elems, bool pool_on_host,
                             hipStream_t st) {
  const int chunks = row_elems * 2 / 16;
#define LS_GATHER(DST, HOST)                                                                  \
  hipLaunchKernelGGL((k_hot_gather<DST, HOST>), dim3(kGatherWGPerReq, B), dim3(256), 0, st,     \
                     miss_pos, n_miss, miss_dst, (const uint4*)pool, (uint4*)hot, hot_slots,    \
                     max_ctx, K, chunks)
  if (miss_dst) {
    if (pool_on_host) LS_GATHER(true, true); else LS_GATHER(true, false);
  } else {
    if (pool_on_host) LS_GATHER(false, true); else LS_GATHER(false, false);
  }
#undef LS_GATHER
  return hipGetLastError();
}

}  // namespace ls
