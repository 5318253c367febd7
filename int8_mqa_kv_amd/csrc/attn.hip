// Decode and append attention over the paged int8 multi-query KV cache, for
// gfx950 (MI355X).
//
// What is computed: each query row (one head of one token of one layer)
// attends the cached keys of its layer's KV slot in [lo, p] (p its position,
// lo = p - W + 1 for a local layer with window W, else 0):
//   out = sum_j softmax_j(scale * q . khat_j) vhat_j,  khat = sK * codeK,
//   vhat = sV * codeV
// ("Como funciona a inferência de IA", section "Por que o cache KV existe";
// "Character.AI: inference optimization", section 03 table: one K/V head for
// all query heads, local layers with a 1024 horizon, KV shared across layers;
// section 05: int8 KV).
//
// How, on CDNA4:
//  * One wavefront carries up to 32 query rows that read the same keys (all
//    heads of a layer: multi-query attention means every head scores against
//    the one KV head, so K/V are read once for all of them).
//  * Keys are processed two pages (32 keys) at a time.  Every matrix-core
//    operand is one contiguous 16-byte lane load of a page record
//    (layout.hpp); decode streams pages HBM -> LDS with gfx950's direct
//    global -> LDS loads.
//  * S^T = K.Q^T and O^T += V^T.P^T both run on fp16 matrix cores
//    (16x16x32, fp32 accumulate).  K and V codes become exact fp16 values
//    c + 1152 with two byte permutes per four codes; the bias is removed
//    through the score accumulator's starting value (-1152 * sum of the q
//    row) and, for PV, through a product of the same P with an all-ones
//    operand.  q rows are scaled by a power of two into fp16's range, where a
//    bf16 element is exact (an fp32 element is carried as two fp16 terms).
//    The S^T tile a lane receives (4 keys of one row) is exactly the P^T
//    operand it needs, so the softmax stays in registers.
//  * P*sV is scaled by a power of two tied to the largest V scale seen so
//    far and carried as two fp16 terms (hi + lo, within 2^-22 of it), so the
//    output keeps about 21 bits of every weight.  The remaining roundings are
//    fp32 sums (the code bias included).
//  * Online softmax in the log2 domain (v_exp_f32) with a lazily moved
//    reference maximum per row.
//  * Decode splits long contexts into chunks (flash-decoding style): the
//    wavefronts of a workgroup take consecutive pages and are merged through
//    LDS; the chunks of one sequence publish partial records and the last one
//    to arrive merges them, inside the same kernel.
#include "internal.hpp"

namespace mqa {

constexpr int kNoExp = -100000;

template <int D>
struct Geo {
  static constexpr int CH = D / 4;       // channels per lane group
  static constexpr int KSTEPS = D / 32;  // matrix-core steps over channels
  static constexpr int KLOADS = D / 64;  // 16-byte K loads per lane per page
  static constexpr int VT = D / 16;      // channel tiles of the PV product
  static constexpr int VLOADS = D / 64;  // 16-byte V loads per lane per page
};

template <int D>
struct PageRegs {
  u32x4 k[Geo<D>::KLOADS];
  u32x4 v[Geo<D>::VLOADS];
  f32x4 sk, sv;
};

template <int D>
__device__ __forceinline__ void load_page(PageRegs<D>& r, const uint8_t* rec, int lane, int lg) {
#pragma unroll
  for (int h = 0; h < Geo<D>::KLOADS; ++h)
    r.k[h] = *reinterpret_cast<const u32x4*>(rec + h * 1024 + lane * 16);
#pragma unroll
  for (int h = 0; h < Geo<D>::VLOADS; ++h)
    r.v[h] = *reinterpret_cast<const u32x4*>(rec + 16 * D + h * 1024 + lane * 16);
  r.sk = *reinterpret_cast<const f32x4*>(rec + 32 * D + lg * 16);
  r.sv = *reinterpret_cast<const f32x4*>(rec + 32 * D + 64 + lg * 16);
}

template <int D>
__device__ __forceinline__ void zero_page(PageRegs<D>& r) {
#pragma unroll
  for (int h = 0; h < Geo<D>::KLOADS; ++h) r.k[h] = u32x4{0, 0, 0, 0};
#pragma unroll
  for (int h = 0; h < Geo<D>::VLOADS; ++h) r.v[h] = u32x4{0, 0, 0, 0};
  r.sk = f32x4{0, 0, 0, 0};
  r.sv = f32x4{0, 0, 0, 0};
}

// ---------------------------------------------------------------------------
// Query operands
// ---------------------------------------------------------------------------
// A query row is scaled by 2^(15-E) (E: the exponent of its largest |element|,
// so the largest scaled element lies in [2^14, 2^15)) and held as fp16
// matrix-core operands.  A bf16 element keeps all its bits (fp16 has three
// more, and only elements below 2^-28 of the row's largest fall out of
// fp16's normal range); an fp32 element is split into two fp16 terms.
template <int D, int QS, int NRT>
struct QOps {
  static constexpr int NQ = QS == 1 ? 1 : 2;  // fp16 terms per element
  static constexpr int STEPS = D / 32;        // 16x16x32 steps over the channels
  f16x8 qf[NRT][NQ][STEPS];  // lane (i, g): row 16n+i, channels g*D/4 + 8k .. +7 at step k
  float bias[NRT];  // -kCodeBias * (sum of the row's fp16 terms): start of every score sum
  float crow[NRT];  // 2^(E-15) * scale * log2(e): undoes the row's power-of-two scale
};

// The fp16 terms of PER elements of one query row, already scaled by a power
// of two, and their sum in fp32 (this lane's share of the bias).
template <int PER, int NQ>
__device__ __forceinline__ float q_terms(const float (&x)[PER], float sc, _Float16 (&t)[NQ][PER]) {
  float sum = 0.0f;
#pragma unroll
  for (int e = 0; e < PER; e += 2) {
    const float y0 = x[e] * sc, y1 = x[e + 1] * sc;
    if constexpr (NQ == 1) {
      t[0][e] = (_Float16)y0;
      t[0][e + 1] = (_Float16)y1;
      sum += (float)t[0][e] + (float)t[0][e + 1];
    } else {
      f16x2 hi, lo;
      split_f16x2(y0, y1, hi, lo);
      t[0][e] = hi[0];
      t[0][e + 1] = hi[1];
      t[1][e] = lo[0];
      t[1][e + 1] = lo[1];
      sum += ((float)hi[0] + (float)lo[0]) + ((float)hi[1] + (float)lo[1]);
    }
  }
  return sum;
}

// Exponent E of a row's largest |element| a (a in [2^(E-1), 2^E)); 0 for an
// all-zero row.  E >= -100 keeps 2^(15-E) finite for absurdly small rows.
__device__ __forceinline__ int q_row_exp(float a) {
  return a > 0.0f ? max(frexp_exp(a), -100) : 0;
}

// Raw query registers of one wavefront: rows 16n + li, channels lg*CH .. +CH.
template <int D, int QS, int NRT>
struct QRaw {
  static constexpr int N = (Geo<D>::CH * (QS == 1 ? 2 : 4)) / 16;  // 16-byte loads per row tile
  u32x4 w[NRT][N];
};

// Issue the loads of the block's query rows (row r starts r*D elements after
// qrow0).  Lanes of rows beyond nrows re-read the last row (convert_q zeroes
// them), so that no load depends on a branch or a select.
template <int D, int QS, int NRT>
__device__ __forceinline__ void load_q_raw(QRaw<D, QS, NRT>& r, const void* __restrict__ qrow0,
                                           int nrows, int li, int lg) {
  constexpr int CH = Geo<D>::CH;
  constexpr int esz = QS == 1 ? 2 : 4;
#pragma unroll
  for (int n = 0; n < NRT; ++n) {
    const int row = min(16 * n + li, nrows - 1);
    const uint8_t* p = static_cast<const uint8_t*>(qrow0) + ((int64_t)row * D + lg * CH) * esz;
#pragma unroll
    for (int i = 0; i < QRaw<D, QS, NRT>::N; ++i)
      r.w[n][i] = *reinterpret_cast<const u32x4*>(p + 16 * i);
  }
}

// Turn the raw rows into fp16 matrix-core operands.  Lane (i, g) owns row i's
// channels g*CH .. g*CH+CH-1, which are exactly its B-operand elements of the
// STEPS steps (8 per step, in order).
template <int D, int QS, int NRT>
__device__ __forceinline__ void convert_q(QOps<D, QS, NRT>& o, const QRaw<D, QS, NRT>& r,
                                          float scale_log2, int nrows, int li) {
  constexpr int CH = Geo<D>::CH;
  constexpr int NQ = QOps<D, QS, NRT>::NQ;
#pragma unroll
  for (int n = 0; n < NRT; ++n) {
    const bool live = 16 * n + li < nrows;
    float x[CH];
    if constexpr (QS == 1) {
#pragma unroll
      for (int i = 0; i < QRaw<D, QS, NRT>::N; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[8 * i + 2 * e] = bitcast<float>(r.w[n][i][e] << 16);
          x[8 * i + 2 * e + 1] = bitcast<float>(r.w[n][i][e] & 0xffff0000u);
        }
    } else {
#pragma unroll
      for (int i = 0; i < QRaw<D, QS, NRT>::N; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) x[4 * i + e] = bitcast<float>(r.w[n][i][e]);
    }
#pragma unroll
    for (int c = 0; c < CH; ++c) x[c] = live ? x[c] : 0.0f;
    float a = 0.0f;
#pragma unroll
    for (int c = 0; c < CH; ++c) a = fmaxf(a, fabsf(x[c]));
    const int E = q_row_exp(row_max4(a));
    _Float16 t[NQ][CH];
    const float sum = row_sum4(q_terms<CH, NQ>(x, ldexp2(1.0f, 15 - E), t));
    o.crow[n] = ldexp2(scale_log2, E - 15);
    o.bias[n] = -kCodeBias * sum;
#pragma unroll
    for (int p = 0; p < NQ; ++p)
#pragma unroll
      for (int k = 0; k < QOps<D, QS, NRT>::STEPS; ++k)
#pragma unroll
        for (int e = 0; e < 8; ++e) o.qf[n][p][k][e] = t[p][8 * k + e];
  }
}

// Lazy softmax reference: a row's reference max only moves when a block's max
// exceeds it by more than kTau (log2 units), so p = exp2(sigma - m_ref) stays
// below 2^kTau and most blocks skip rescaling the accumulators.  The weights
// are formed already multiplied by 2^lpv, lpv = kPvBias - ev, through the
// exponent's offset (every V scale seen is below 2^ev; ev is set
// kVExpHeadroom above the largest one's exponent whenever it moves, so that
// later blocks rarely move it; lpv = 0 while no V scale was seen): P*sV then
// stays below 2^14 as an fp16 operand, and the running sum l is kept in the
// same units until the key loop ends.  Both
// conditions are tested first against thresholds cached when the reference
// last moved (a key's score times its scale, and a V scale, each compared in
// its own lane); only a block that passes one works out row maxima across
// lanes and the new references.  (Where the threshold test and the reference
// test round differently, p may exceed 2^kTau by a rounding, or a block takes
// the full path and moves nothing; results stay deterministic.)
constexpr float kTau = 8.0f;
constexpr int kPvBias = 14 - 8;
constexpr int kVExpHeadroom = 2;
// Smallest V exponent tracked: keeps 2^lpv, and l in its units, finite for
// absurdly small scales (a V scale below 2^-64 contributes below 2^-57 to any
// output).
constexpr int kMinVExp = -64;

// ---------------------------------------------------------------------------
// One wavefront's running softmax state over its keys
// ---------------------------------------------------------------------------
template <int D, int NRT>
struct WaveState {
  f32x4 acc[NRT][Geo<D>::VT];  // O^T tiles: lane (i, g) holds channels 16t+4g..+3 of row i
  f32x4 psum[NRT];             // sum of the P operand over keys, row i (all 4 equal)
  float m[NRT];                // running max (log2 domain), equal on a row's 4 lanes
  float l[NRT];                // this lane's part of the row's running sum, in units of
                               // 2^lpv during the key loop (plain after finish())
  int ev;                      // every V scale seen is below 2^ev, set kVExpHeadroom above
                               // the largest one's exponent when it moves (kNoExp: none)
  // Cached from the last time the reference or the V exponent moved: a key
  // scale times score above thr[n] moves row n's reference; a V scale at or
  // above ev_thr = 2^ev moves the exponent; off[n] = lpv - m (lpv for
  // m = -inf) is the exponent's offset.
  float thr[NRT], off[NRT];
  float ev_thr;

  __device__ __forceinline__ void init() {
#pragma unroll
    for (int n = 0; n < NRT; ++n) {
      m[n] = kNegInf;
      l[n] = 0.0f;
      thr[n] = kNegInf;
      off[n] = 0.0f;
      psum[n] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int t = 0; t < Geo<D>::VT; ++t) acc[n][t] = f32x4{0, 0, 0, 0};
    }
    ev = kNoExp;
    ev_thr = 0.0f;
  }
  // The accumulators hold P.(V codes + kCodeBias): take kCodeBias * sum(P)
  // out and restart that sum.  Done every kRebiasBlocks blocks, not only at
  // the end, so that the accumulators stay near the size of the result: the
  // bias part grows with every block, and over a long key range its fp32
  // rounding would otherwise outgrow an output that is an average over
  // thousands of keys.
  __device__ __forceinline__ void rebias() {
#pragma unroll
    for (int n = 0; n < NRT; ++n) {
#pragma unroll
      for (int t = 0; t < Geo<D>::VT; ++t)
#pragma unroll
        for (int k = 0; k < 4; ++k)
          acc[n][t][k] = __builtin_fmaf(-kCodeBias, psum[n][k], acc[n][t][k]);
      psum[n] = f32x4{0, 0, 0, 0};
    }
  }
  // After the last key: the remaining bias comes out; l returns from units
  // of 2^lpv.
  __device__ __forceinline__ void finish() {
    rebias();
    const float u = ev == kNoExp ? 1.0f : ldexp2(1.0f, ev - kPvBias);
#pragma unroll
    for (int n = 0; n < NRT; ++n) l[n] *= u;
  }
};
constexpr int kRebiasBlocks = 32;

// Attend the 32 keys of two consecutive logical pages.  pos0 is the position
// of the first page's first token.  MASKED blocks (some key outside [lo, hi)
// or on a page that is not ok) select every masked key away, so poison bytes
// in those keys are never used; interior blocks skip the selects.
template <int D, int QS, int NRT, bool MASKED>
__device__ __forceinline__ void attend_block(WaveState<D, NRT>& st, const QOps<D, QS, NRT>& q,
                                             const PageRegs<D>& p0, const PageRegs<D>& p1,
                                             bool ok0, bool ok1, int pos0, int lo, int hi,
                                             int lg) {
  constexpr int STEPS = QOps<D, QS, NRT>::STEPS, NQ = QOps<D, QS, NRT>::NQ;
  // S^T for both pages on the fp16 matrix cores: 8 stored K bytes (token i,
  // channels g*D/4 + 8k ..) are lane (i, g)'s A operand of step k as fp16
  // c + kCodeBias; the q row is B.  Each sum starts at -kCodeBias * (the
  // row's sum), which takes the bias back out.  Lane (i, g) gets the scores
  // of keys 4g..4g+3 for row i.
  f32x4 s[NRT][2];
#pragma unroll
  for (int n = 0; n < NRT; ++n)
#pragma unroll
    for (int u = 0; u < 2; ++u) s[n][u] = f32x4{q.bias[n], q.bias[n], q.bias[n], q.bias[n]};
#pragma unroll
  for (int k = 0; k < STEPS; ++k)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const PageRegs<D>& P = u ? p1 : p0;
      const int h = k >> 1, w = 2 * (k & 1);
      const f16x8 kop = codes_to_f16x8_biased(P.k[h][w], P.k[h][w + 1]);
#pragma unroll
      for (int n = 0; n < NRT; ++n)
#pragma unroll
        for (int t = 0; t < NQ; ++t) s[n][u] = mma16(kop, q.qf[n][t][k], s[n][u]);
    }

  bool valid[2][4];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int pos = pos0 + 16 * u + 4 * lg + r;
      valid[u][r] = !MASKED || ((u ? ok1 : ok0) && pos >= lo && pos < hi);
    }

  // t = score * key scale (-inf for a masked key); the row's factor crow
  // (> 0) is applied in the exponent's FMA.  First the cheap test: does any
  // key move a row's reference (t above the row's cached threshold) or the V
  // exponent (a valid V scale at or above 2^ev)?  Only then (wave-uniform,
  // rare after a row's first blocks) are the row maxima, the new references
  // and the rescale worked out.
  float t[NRT][2][4];
  float lmax[NRT];
  float vmax = 0.0f;
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float sv = (u ? p1.sv : p0.sv)[r];
      vmax = fmaxf(vmax, MASKED ? (valid[u][r] ? sv : 0.0f) : sv);
    }
  bool moves = vmax >= st.ev_thr;
#pragma unroll
  for (int n = 0; n < NRT; ++n) {
    float mt = kNegInf;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float x = s[n][u][r] * (u ? p1.sk : p0.sk)[r];
        t[n][u][r] = MASKED ? (valid[u][r] ? x : kNegInf) : x;
        mt = fmaxf(mt, t[n][u][r]);
      }
    lmax[n] = mt;
    moves |= mt > st.thr[n];
  }
  if (__builtin_amdgcn_ballot_w64(moves) != 0) {  // wave-uniform
    // Largest valid V scale of the block -> running exponent.
    const float vm = row_max4(vmax);
    int ev_new = st.ev;
    if (vm > 0.0f) ev_new = max(ev_new, max(frexp_exp(vm) + kVExpHeadroom, kMinVExp));
    const int lpv_old = st.ev == kNoExp ? 0 : kPvBias - st.ev;
    const int lpv = ev_new == kNoExp ? 0 : kPvBias - ev_new;
    const int dexp = lpv - lpv_old;  // the units of acc, psum and l change by 2^dexp
    st.ev = ev_new;
    st.ev_thr = ev_new == kNoExp ? 0.0f : ldexp2(1.0f, ev_new);
    float alpha[NRT];
    bool rescale = false, held = false;
#pragma unroll
    for (int n = 0; n < NRT; ++n) {
      const float mt = row_max4(lmax[n]);
      const float mx = mt == kNegInf ? kNegInf : mt * q.crow[n];
      const bool move = mx > st.m[n] + kTau;  // also true for the first valid block
      const float m_new = move ? mx : st.m[n];
      // a row whose reference is still -inf has seen no valid key: its sums
      // are zero and need no rescale
      const bool had = st.m[n] != kNegInf;
      alpha[n] = move ? fast_exp2(st.m[n] - m_new) : 1.0f;  // exp2(-inf) = 0
      rescale |= move && had;
      held |= had;
      st.off[n] = m_new == kNegInf ? (float)lpv : (float)lpv - m_new;
      st.thr[n] = m_new == kNegInf ? kNegInf : (m_new + kTau) * __builtin_amdgcn_rcpf(q.crow[n]);
      st.m[n] = m_new;
    }
    // rescale only when a row with sums moved its reference, or the V
    // exponent grew while some row had sums (wave-uniform branch)
    if (__builtin_amdgcn_ballot_w64(rescale) != 0 ||
        (dexp != 0 && __builtin_amdgcn_ballot_w64(held) != 0)) {
#pragma unroll
      for (int n = 0; n < NRT; ++n) {
        const float f = ldexp2(alpha[n], dexp);
#pragma unroll
        for (int t = 0; t < Geo<D>::VT; ++t) st.acc[n][t] *= f;
        st.psum[n] *= f;
        st.l[n] *= f;
      }
    }
  }
  float off[NRT];
#pragma unroll
  for (int n = 0; n < NRT; ++n) off[n] = st.off[n];

  // P*sV as two fp16 terms, hi and lo (hi + lo within 2^-22 of it)
  f16x8 ph[NRT], pl[NRT];
#pragma unroll
  for (int n = 0; n < NRT; ++n) {
    float ps;
    float pv[8];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        // p * 2^lpv
        const float pr = fast_exp2(__builtin_fmaf(t[n][u][r], q.crow[n], off[n]));
        ps = u == 0 && r == 0 ? pr : ps + pr;
        const float x = pr * (u ? p1.sv : p0.sv)[r];
        pv[4 * u + r] = MASKED ? (valid[u][r] ? x : 0.0f) : x;
      }
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      f16x2 hi, lo;
      split_f16x2(pv[e], pv[e + 1], hi, lo);
      ph[n][e] = hi[0];
      ph[n][e + 1] = hi[1];
      pl[n][e] = lo[0];
      pl[n][e + 1] = lo[1];
    }
    st.l[n] += ps;
  }
  // V codes enter as c + kCodeBias (two byte permutes per four codes); the
  // matching sum of P comes from products with an all-ones operand, so it
  // uses the very fp16 terms the accumulators saw.
#pragma unroll
  for (int t = 0; t < Geo<D>::VT; ++t) {
    const int h = t >> 2, dw = t & 3;
    const f16x8 vop = codes_to_f16x8_biased(p0.v[h][dw], p1.v[h][dw]);
#pragma unroll
    for (int n = 0; n < NRT; ++n) st.acc[n][t] = mma16(vop, ph[n], st.acc[n][t]);
#pragma unroll
    for (int n = 0; n < NRT; ++n) st.acc[n][t] = mma16(vop, pl[n], st.acc[n][t]);
  }
  const _Float16 one = 1.0f;
  const f16x8 ones = {one, one, one, one, one, one, one, one};
#pragma unroll
  for (int n = 0; n < NRT; ++n) st.psum[n] = mma16(ones, ph[n], st.psum[n]);
#pragma unroll
  for (int n = 0; n < NRT; ++n) st.psum[n] = mma16(ones, pl[n], st.psum[n]);
}

template <int D, int QS, int NRT>
__device__ __forceinline__ void attend_block_any(WaveState<D, NRT>& st, const QOps<D, QS, NRT>& q,
                                                 const PageRegs<D>& p0, const PageRegs<D>& p1,
                                                 bool ok0, bool ok1, int pos0, int lo, int hi,
                                                 int lg) {
  const bool masked = !(ok0 && ok1 && pos0 >= lo && pos0 + 2 * kPageTokens <= hi);
  if (masked)
    attend_block<D, QS, NRT, true>(st, q, p0, p1, ok0, ok1, pos0, lo, hi, lg);
  else
    attend_block<D, QS, NRT, false>(st, q, p0, p1, ok0, ok1, pos0, lo, hi, lg);
}

__device__ __forceinline__ int clamp_ctx(int ctx, int max_context, int max_pages) {
  const int cap = (int)min<int64_t>(max_context, (int64_t)max_pages * kPageTokens);
  return min(max(ctx, 0), cap);
}

// One wavefront's share of a decode sequence's key range [lo, hi): the
// range's pages split over chunks of at least 16 pages (two per wavefront)
// where the range allows, then evenly over the W wavefronts of the chunk.
// A windowed range moves with the context length, so its chunks split the
// range itself.  A global range always starts at key 0, so its chunk
// boundaries are placed on the longest range the launch allows (ctx_cap
// keys): they, and the pages every wavefront reads, then do not depend on
// the sequence's own length, and a shorter sequence simply fills fewer
// chunks (nch of them).  The critical path -- a chunk of the longest range --
// is the same either way.
template <int W>
struct WaveSpan {
  int lo, hi;      // keys
  int p_last;      // last page of the range
  int nch;         // chunks of the range that hold pages
  int pbeg, pend;  // this wavefront's pages [pbeg, pend)

  __device__ __forceinline__ WaveSpan(int ctx, int ctx_cap, int window, int nchunk, int chunk,
                                      int wv) {
    hi = ctx;
    lo = window > 0 ? max(0, ctx - window) : 0;
    const int p_first = lo >> 4;
    p_last = (hi - 1) >> 4;
    const int np = p_last - p_first + 1;
    // (the host bounds max_context by 2^22 keys and the chunks by 2^11:
    // np <= 2^18 + 1 pages, so the products stay within 32 bits)
    const int npb = window > 0 ? np : max((ctx_cap + kPageTokens - 1) / kPageTokens, 1);
    const int nchb = min(nchunk, max(1, (npb + 2 * W - 1) / (2 * W)));
    nch = window > 0 ? nchb : (int)(((uint32_t)(np * nchb) + npb - 1) / (uint32_t)npb);
    const int cbeg = p_first + (int)((uint32_t)(chunk * npb) / (uint32_t)nchb);
    const int npc = p_first + (int)((uint32_t)((chunk + 1) * npb) / (uint32_t)nchb) - cbeg;
    pbeg = cbeg + wv * npc / W;
    pend = max(pbeg, min(cbeg + (wv + 1) * npc / W, p_first + np));
  }
};

// XCD-aware flat index: hardware workgroup x runs on XCD x % 8, so give each
// XCD a contiguous range of logical work (gridDim.x is a multiple of 8).
// The grid is total rounded up to a multiple of 8 (padded_grid); taking its
// size from the launch's own total keeps the read in the same batch as the
// other kernel arguments.
__device__ __forceinline__ int swizzled_block(int total) {
  const int nx = (total + 7) & ~7, x = blockIdx.x;
  return (x & 7) * (nx >> 3) + (x >> 3);
}

// ---------------------------------------------------------------------------
// Decode: one workgroup = one (row block, sequence, chunk of pages)
// ---------------------------------------------------------------------------
struct DecodeWork {
  DecodeGroup g;
  RowBlock rb;
  int rbl, seq, chunk;
};

// x / d and x % d (x < 2^31, d >= 1, recip = recip_of(d))
__device__ __forceinline__ void udiv_recip(uint32_t x, uint32_t d, uint32_t recip, uint32_t& q,
                                           uint32_t& r) {
  q = __umulhi(x, recip);
  r = x - q * d;
  if (r >= d) {
    ++q;
    r -= d;
  }
}

// The workgroup's (group, row block, chunk, sequence).  Kernel arguments are
// read with scalar loads whose round trips add up when one address depends on
// another; see decode_work for how the usual launch avoids that.
// A kernel's first argument, read in place in the kernel-argument segment
// (the first argument sits at offset 0).  Indexing a by-value argument with a
// computed index makes the compiler copy the whole struct out of that segment
// first; reading through this pointer does not.
template <typename T>
__device__ __forceinline__ const T* first_kernel_arg() {
  // (a C-style cast: from the constant address space to a generic pointer)
  return (const T*)__builtin_amdgcn_kernarg_segment_ptr();
}

__device__ __forceinline__ DecodeWork decode_work(const DecodeArgs& a, int w) {
  DecodeWork d;
  uint32_t q, r;
  // The usual launch -- one (slot, window) group of at most four row blocks
  // -- finds every field at a fixed offset, so it is worked out first, from
  // one round of loads issued together; any other launch redoes it below.
  const DecodeGroup g = a.groups[0];
  const RowBlock r0 = a.rbs[0], r1 = a.rbs[1], r2 = a.rbs[2], r3 = a.rbs[3];
  d.g = g;
  udiv_recip((uint32_t)(w - g.wg_begin), (uint32_t)g.num_rb, g.rb_recip, q, r);
  d.rbl = (int)r;
  d.rb = r == 0 ? r0 : r == 1 ? r1 : r == 2 ? r2 : r3;
  udiv_recip(q, (uint32_t)g.nchunk, g.ch_recip, q, r);
  d.chunk = (int)r;
  d.seq = (int)q;
  if (a.num_groups == 1 && g.num_rb <= 4) return d;
  // Any other launch: find the group, then read it and the row block at
  // computed offsets (volatile: these reads stay apart from the ones above).
  const volatile DecodeArgs* ka = first_kernel_arg<volatile DecodeArgs>();
  const int ng = a.num_groups;
  int gi = 0;
  while (gi + 1 < ng && w >= ka->groups[gi + 1].wg_begin) ++gi;
  const volatile DecodeGroup& vg = ka->groups[gi];
  d.g.slot = vg.slot;
  d.g.window = vg.window;
  d.g.first_rb = vg.first_rb;
  d.g.num_rb = vg.num_rb;
  d.g.nchunk = vg.nchunk;
  d.g.wg_begin = vg.wg_begin;
  d.g.ws_begin = vg.ws_begin;
  d.g.merge_begin = vg.merge_begin;
  d.g.writes_new_kv = vg.writes_new_kv;
  d.g.nontemporal = vg.nontemporal;
  d.g.rb_recip = vg.rb_recip;
  d.g.ch_recip = vg.ch_recip;
  udiv_recip((uint32_t)(w - d.g.wg_begin), (uint32_t)d.g.num_rb, d.g.rb_recip, q, r);
  d.rbl = (int)r;
  udiv_recip(q, (uint32_t)d.g.nchunk, d.g.ch_recip, q, r);
  d.chunk = (int)r;
  d.seq = (int)q;
  const volatile RowBlock& vr = ka->rbs[d.g.first_rb + d.rbl];
  d.rb.layer = vr.layer;
  d.rb.head0 = vr.head0;
  d.rb.nrows = vr.nrows;
  return d;
}

// ---------------------------------------------------------------------------
// Page staging through LDS (gfx950 global -> LDS loads: lane l's 16 bytes land
// at base + 16*l, which is exactly the page layout, so a page record moves
// from HBM into LDS without passing through registers).
// ---------------------------------------------------------------------------
// LDS slot of one page: the record plus 128 bytes of padding that the
// branch-free scale load below may write into.
template <int D>
constexpr int lds_slot_bytes() { return page_bytes(D) + 128; }

// One 1 KiB piece of a record at byte OFF: the instruction offset applies to
// both the global and the LDS address, so every piece of a page shares one
// address computation and one LDS base.
// Cache policy of a page load: 0, or the non-temporal bit for pages that
// nothing reuses soon (the planner's choice per group).
constexpr int kCpolNonTemporal = 2;

template <int OFF, int CPOL>
__device__ __forceinline__ void dma_kib(const uint8_t* lane_src, uint8_t* lds_slot) {
  __builtin_amdgcn_global_load_lds(lane_src, lds_slot, 16, OFF, CPOL);
}

template <int D, int CPOL = 0>
__device__ __forceinline__ void dma_page(uint8_t* lds_slot, const uint8_t* __restrict__ rec,
                                         int lane) {
  const uint8_t* src = rec + lane * 16;
  dma_kib<0, CPOL>(src, lds_slot);
  dma_kib<1024, CPOL>(src, lds_slot);
  if constexpr (D == 128) {
    dma_kib<2048, CPOL>(src, lds_slot);
    dma_kib<3072, CPOL>(src, lds_slot);
  }
  // the 128 bytes of fp32 scales: 4 bytes per lane; lanes 32..63 re-read the
  // last scale and land in the slot's padding (no branch, no exec change)
  __builtin_amdgcn_global_load_lds(rec + 32 * D + 4 * min(lane, 31), lds_slot + 32 * D, 4, 0, CPOL);
}

template <int D>
__device__ __forceinline__ void lds_page(PageRegs<D>& r, const uint8_t* lds_slot, int lane,
                                         int lg) {
#pragma unroll
  for (int h = 0; h < Geo<D>::KLOADS; ++h)
    r.k[h] = *reinterpret_cast<const u32x4*>(lds_slot + h * 1024 + lane * 16);
#pragma unroll
  for (int h = 0; h < Geo<D>::VLOADS; ++h)
    r.v[h] = *reinterpret_cast<const u32x4*>(lds_slot + 16 * D + h * 1024 + lane * 16);
  r.sk = *reinterpret_cast<const f32x4*>(lds_slot + 32 * D + lg * 16);
  r.sv = *reinterpret_cast<const f32x4*>(lds_slot + 32 * D + 64 + lg * 16);
}

// Decode workgroup LDS: q operands converted once for all wavefronts, per-row
// softmax scales, the wavefronts' softmax statistics and the cross-workgroup
// arrival flag, kept apart from the page rings (written by global -> LDS
// loads) so that the compiler can tell them apart.
template <int D, int QS, int NRT, int W>
struct DecodeQLds {
  f16x8 qf[NRT][QOps<D, QS, NRT>::NQ][QOps<D, QS, NRT>::STEPS][64];
  float crow[32];
  float qb[32];
  float m[W][32];
  float l[W][32];
  int ev[W];
};
// Each wavefront's ring of RB blocks of two pages.  Once its pages are
// consumed, a wavefront dumps its accumulators into its own ring for the
// cross-wavefront merge.
template <int D, int W, int RB>
struct alignas(16) DecodeRingLds {
  uint8_t ring[W][2 * RB][lds_slot_bytes<D>()];
};

// s_waitcnt immediate for "at most n vector-memory operations outstanding"
// (expcnt and lgkmcnt left at their maxima; vmcnt's 6 bits are split 4 + 2).
constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 15) | (((n >> 4) & 3) << 14); }
// s_waitcnt immediate for "no LDS operation outstanding" (vmcnt, expcnt at max).
constexpr int kLgkmZero = 0xC07F;

// Workgroup barrier that publishes this wavefront's LDS writes but leaves its
// global -> LDS page loads in flight (__syncthreads() would wait for every
// outstanding memory operation first).  The empty asm statements keep the
// compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(kLgkmZero);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The block's query rows staged into fp16 matrix-core operands in LDS, once
// for all W wavefronts: wavefront w takes rows 4w..4w+3, 4w+4W.., 16 lanes per
// row, D/16 channels per lane.  The raw rows travel global -> LDS first
// (StageQ::issue, into the wavefront's own staging area): such loads are
// issued where they stand, while ordinary loads whose results are used only
// past the kernel's early exits would be sunk below them by the compiler.
// StageQ::store then converts them once they have landed.
template <int D, int QS, int NRT, int W>
struct StageQ {
  static constexpr int PER = D / 16;                       // channels per lane
  static constexpr int PASSES = (16 * NRT + 4 * W - 1) / (4 * W);
  static constexpr int ESZ = QS == 1 ? 2 : 4;
  static constexpr int LB = PER * ESZ;                     // raw bytes per lane per pass
  static constexpr int CB = LB >= 16 ? 16 : 4;             // bytes per global -> LDS load
  static constexpr int NC = LB / CB;                       // loads per lane per pass
  static constexpr int STAGE_BYTES = PASSES * NC * 64 * CB;
  static constexpr int WORDS = LB / 4;                     // dwords per lane per pass

  __device__ __forceinline__ void issue(uint8_t* stage, const void* __restrict__ qrow0, int nrows,
                                        int wv, int lane) const {
    const int sub = lane >> 4, part = lane & 15;
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
      if (wv * 4 + ps * 4 * W >= 16 * NRT) break;  // wave-uniform: no rows to stage
      const int row = wv * 4 + ps * 4 * W + sub;
      const int rr = row < nrows ? row : 0;
      const uint8_t* src = static_cast<const uint8_t*>(qrow0) + ((int64_t)rr * D + part * PER) * ESZ;
#pragma unroll
      for (int k = 0; k < NC; ++k) {
        if constexpr (CB == 16)
          __builtin_amdgcn_global_load_lds(src + k * 16, stage + (ps * NC + k) * 64 * 16, 16, 0, 0);
        else
          __builtin_amdgcn_global_load_lds(src + k * 4, stage + (ps * NC + k) * 64 * 4, 4, 0, 0);
      }
    }
  }

  // dword w of this lane's raw row data of pass ps
  __device__ __forceinline__ uint32_t raw(const uint8_t* stage, int ps, int w, int lane) const {
    const int k = (4 * w) / CB;
    return *reinterpret_cast<const uint32_t*>(stage + (ps * NC + k) * 64 * CB + lane * CB +
                                              (4 * w) % CB);
  }

  template <typename Lds>
  __device__ __forceinline__ void store(Lds& sm, const uint8_t* stage, int nrows,
                                        float scale_log2, int wv, int lane) const {
    constexpr int CH = Geo<D>::CH;
    constexpr int NQ = QOps<D, QS, NRT>::NQ;
    const int sub = lane >> 4, part = lane & 15;
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
      // wavefronts past the block's rows (W = 8 with 16 rows) have nothing to
      // stage and must not write (they would clobber another row's operands)
      if (wv * 4 + ps * 4 * W >= 16 * NRT) break;  // wave-uniform
      const int row = wv * 4 + ps * 4 * W + sub;
      const bool live = row < nrows;
      uint32_t rw[WORDS];
#pragma unroll
      for (int e = 0; e < WORDS; ++e) rw[e] = raw(stage, ps, e, lane);
      float x[PER];
      if constexpr (QS == 1) {
#pragma unroll
        for (int e = 0; e < PER / 2; ++e) {
          x[2 * e] = bitcast<float>(rw[e] << 16);
          x[2 * e + 1] = bitcast<float>(rw[e] & 0xffff0000u);
        }
      } else {
#pragma unroll
        for (int e = 0; e < PER; ++e) x[e] = bitcast<float>(rw[e]);
      }
      float a = 0.0f;
#pragma unroll
      for (int e = 0; e < PER; ++e) {
        x[e] = live ? x[e] : 0.0f;
        a = fmaxf(a, fabsf(x[e]));
      }
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) a = fmaxf(a, __shfl_xor(a, off));
      const int E = q_row_exp(a);
      _Float16 t[NQ][PER];
      float sum = q_terms<PER, NQ>(x, ldexp2(1.0f, 15 - E), t);
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) sum += __shfl_xor(sum, off);
      if (part == 0) {
        sm.crow[row] = ldexp2(scale_log2, E - 15);
        sm.qb[row] = -kCodeBias * sum;
      }
      // operand elements of (row, channels c0..c0+PER-1): tile n, lane (li,
      // lg), step k, element e0 of the lane's eight
      const int c0 = part * PER;
      const int n = row >> 4, li = row & 15;
      const int lg = c0 / CH, k = (c0 % CH) >> 3, e0 = c0 & 7;
#pragma unroll
      for (int p = 0; p < NQ; ++p) {
        _Float16* dst = reinterpret_cast<_Float16*>(&sm.qf[n][p][k][16 * lg + li]) + e0;
        if constexpr (PER == 8) {
          *reinterpret_cast<f16x8*>(dst) =
              f16x8{t[p][0], t[p][1], t[p][2], t[p][3], t[p][4], t[p][5], t[p][6], t[p][7]};
        } else {
          static_assert(PER == 4, "channels per lane");
          *reinterpret_cast<f16x2*>(dst) = f16x2{t[p][0], t[p][1]};
          *reinterpret_cast<f16x2*>(dst + 2) = f16x2{t[p][2], t[p][3]};
        }
      }
    }
  }
};

// The current token of a fused decode step ("Como funciona a inferência de
// IA", section "Por que o cache KV existe": a new token's K and V are computed
// once and kept).  Its K and V rows are loaded when the workgroup starts,
// coded to int8 with the pack kernel's arithmetic, written into the LDS copy
// of their page before that page is read (the step never reads the token back
// from HBM) and, by one workgroup per slot, into the pool for later steps.
template <int D, NewKV NK>
struct CurrentToken {
  static constexpr int PER = D / 64;  // channels lane*PER .. lane*PER+PER-1
  float xk[PER], xv[PER];
  int ck[PER], cv[PER];
  float sk, sv;

  __device__ __forceinline__ void load(const void* __restrict__ kp, const void* __restrict__ vp,
                                       int64_t row, int lane) {
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int64_t i = row * D + lane * PER + e;
      if constexpr (NK == NewKV::kBf16) {
        xk[e] = bf16_to_f32(static_cast<const uint16_t*>(kp)[i]);
        xv[e] = bf16_to_f32(static_cast<const uint16_t*>(vp)[i]);
      } else {
        xk[e] = static_cast<const float*>(kp)[i];
        xv[e] = static_cast<const float*>(vp)[i];
      }
    }
  }
  __device__ __forceinline__ void code() {
    const float ak = wave_absmax<PER>(xk), av = wave_absmax<PER>(xv);
    sk = quant_scale(ak);
    sv = quant_scale(av);
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      ck[e] = quant_code(xk[e], ak, sk);
      cv[e] = quant_code(xv[e], av, sv);
    }
  }
  // write the token into a page record (an LDS copy or the pool) as token j
  __device__ __forceinline__ void put(uint8_t* rec, int j, int lane) const {
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int c = lane * PER + e;
      rec[k_code_offset(D, j, c)] = code_byte(ck[e]);
      rec[v_code_offset(D, j, c)] = code_byte(cv[e]);
    }
    if (lane == 0) {
      *reinterpret_cast<float*>(rec + k_scale_offset(D, j)) = sk;
      *reinterpret_cast<float*>(rec + v_scale_offset(D, j)) = sv;
    }
  }
};

// Device-coherent handoff between workgroups.  Agent-scope relaxed atomic
// loads and stores are coherent across the XCDs' separate L2 caches (gfx950
// marks them sc1); pairing them with a wait for the stores' completion before
// the arrival is counted avoids a full L2 write-back fence.
__device__ __forceinline__ void st_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Decode, optionally fused with storing the current token (NK != kNone).
// Per workgroup: stage q; stream this wavefront's pages HBM -> LDS through its
// ring; attend; merge the W wavefronts in one LDS exchange; then either write
// the output (the workgroup covered the whole key range) or publish a partial
// record, count the arrival, and let the chunk that arrives last fold every
// chunk's record in chunk order and write the output.
// W wavefronts per workgroup: 8 (one workgroup per CU), or 4 (two per CU, so
// that launches with few items fill more of the chip); two wavefronts per SIMD
// either way, which the launch bound's second argument states for W = 4.
template <int D, int QS, int NRT, NewKV NK, int W>
__global__ __launch_bounds__(W * 64, 2) void decode_kernel(
    const DecodeArgs a, const void* __restrict__ qp, float* __restrict__ out,
    uint8_t* __restrict__ pool, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ context_lens, float* __restrict__ ws,
    const void* __restrict__ k_new, const void* __restrict__ v_new) {
  constexpr int RB = kDecodeRing;
  constexpr int VT = Geo<D>::VT;
  constexpr int PAIRS = NRT * VT;             // (row tile, channel tile) pairs of the output
  constexpr int PPW = (PAIRS + W - 1) / W;    // pairs per wavefront in the merge
  __shared__ DecodeQLds<D, QS, NRT, W> sm;
  __shared__ DecodeRingLds<D, W, RB> ring;
  static_assert(sizeof(DecodeQLds<D, QS, NRT, W>) + sizeof(DecodeRingLds<D, W, RB>) <= 160 * 1024,
                "LDS");
  static_assert(PAIRS * 64 * sizeof(f32x4) <= sizeof(ring.ring[0]), "accumulator dump");
  constexpr int DMA_PER_BLOCK = 2 * (32 * D / 1024 + 1);
  const int w = swizzled_block(a.total_wgs);
  // (the mapping's reads do not depend on w being in range; leaving first)
  const DecodeWork dw = decode_work(a, w);
  if (w >= a.total_wgs) return;
  const DecodeGroup& g = dw.g;
  const RowBlock& rb = dw.rb;
  const int seq = dw.seq, chunk = dw.chunk;

  const int lane = lane_id(), li = lane & 15, lg = lane >> 4;
  const int wv = threadIdx.x >> 6;
  const int64_t out_row0 = ((int64_t)rb.layer * a.batch + seq) * a.num_q_heads + rb.head0;
  // The query rows do not depend on the context length: their loads go out
  // together with the length's.
  StageQ<D, QS, NRT, W> sq;
  static_assert(StageQ<D, QS, NRT, W>::STAGE_BYTES <= lds_slot_bytes<D>(), "q staging");
  uint8_t* const stage = &ring.ring[wv][0][0];  // free until the first pages are issued
  sq.issue(stage, static_cast<const uint8_t*>(qp) + out_row0 * D * (QS == 1 ? 2 : 4), rb.nrows, wv,
           lane);
  // the current token's rows do not depend on it either
  CurrentToken<D, NK> cur;
  if constexpr (NK != NewKV::kNone)
    cur.load(k_new, v_new, (int64_t)g.slot * a.batch + seq, lane);
  // Nor, as a guess, do the page ids: they are loaded for the span of the
  // longest context the launch allows (exact for a global range; for a
  // windowed one whenever the sequence has that length) together with the
  // length itself, and reloaded below only when the guess was wrong.
  const int ctx_cap = clamp_ctx(a.max_context, a.max_context, a.max_pages);
  const int32_t* table_row = block_table + ((int64_t)g.slot * a.batch + seq) * (int64_t)a.max_pages;
  const WaveSpan<W> guess(ctx_cap, ctx_cap, g.window, g.nchunk, chunk, wv);
  int ids = guess.pbeg + lane < guess.pend ? table_row[guess.pbeg + lane] : -1;
  const int ctx_raw = context_lens[seq];
  // All of the above are in flight together; wait for them here, before the
  // branches below (the compiler would otherwise sink the loads whose values
  // are used only past them, and each would cost a round trip of its own).
  if constexpr (NK != NewKV::kNone) {
#pragma unroll
    for (int e = 0; e < CurrentToken<D, NK>::PER; ++e)
      asm volatile("" ::"v"(cur.xk[e]), "v"(cur.xv[e]));
  }
  asm volatile("" ::"v"(ids), "v"(ctx_raw));
  const int ctx = clamp_ctx(ctx_raw, a.max_context, a.max_pages);
  WaveSpan<W> sp = guess;
  if (ctx != ctx_cap) sp = WaveSpan<W>(ctx, ctx_cap, g.window, g.nchunk, chunk, wv);
  const int lo = sp.lo, hi = sp.hi;

  if (hi <= lo) {  // empty context: zeros (and no current token to store)
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // (the staged q rows land first)
    if (chunk == 0 && wv == 0) {
      for (int n = 0; n < NRT; ++n) {
        const int row = 16 * n + li;
        if (row < rb.nrows)
          for (int t = 0; t < VT; ++t)
            *reinterpret_cast<f32x4*>(out + (out_row0 + row) * D + 16 * t + 4 * lg) =
                f32x4{0, 0, 0, 0};
      }
    }
    return;
  }
  const int nch = sp.nch, p_last = sp.p_last;
  if (chunk >= nch) {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    return;
  }
  // (wave-uniform: in scalar registers, so that the loop's page checks are
  // scalar instructions)
  const int pbeg = __builtin_amdgcn_readfirstlane(sp.pbeg);
  const int pend = __builtin_amdgcn_readfirstlane(sp.pend);
  const uint32_t pool_pages = (uint32_t)min<int64_t>(a.num_pages, 0xFFFFFFFF);
  if (pbeg != guess.pbeg || pend > guess.pend)  // wave-uniform
    ids = pbeg + lane < pend ? table_row[pbeg + lane] : -1;
  auto page_ok = [&](int pi, int& pid) {
    pid = __builtin_amdgcn_readlane(ids, min(max(pi - pbeg, 0), 63));
    return pi < pend && (uint32_t)pid < pool_pages;
  };
  // q is converted before any page load is issued, so that waiting for it
  // does not wait for pages (the ids and the current token's rows, issued
  // after q, are needed right after it anyway).
  // the staged rows (the oldest loads of this wavefront) have landed
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __builtin_amdgcn_sched_barrier(0);
  sq.store(sm, stage, rb.nrows, a.scale_log2, wv, lane);
  __builtin_amdgcn_sched_barrier(0);
  const int tok = (hi - 1) & 15;  // the current token's place in page p_last
  // the block of this wavefront holding page p_last (the range's last), or -1
  const int b_cur = p_last >= pbeg && p_last < pend ? (p_last - pbeg) >> 1 : -1;
  if constexpr (NK != NewKV::kNone) {
    // The wavefront whose pages include p_last codes the current token now.
    // The one workgroup per slot and sequence that keeps it for later steps
    // stores it here, so that the store flies with the first page loads
    // instead of being waited for after the last one.  Every reader of the
    // page, this one included, writes the token into its LDS copy, so loads
    // of that page need not see the store.
    if (b_cur >= 0) {
      cur.code();
      int pid;
      if (g.writes_new_kv && dw.rbl == 0 && page_ok(p_last, pid))
        cur.put(pool + (int64_t)pid * page_bytes(D), tok, lane);
    }
  }
  // branch-free: a page that is out of range or has a bad id loads page 0
  // instead (it exists) and is masked later.  Where the planner finds that
  // nothing reuses the pages soon (one reader, or readers that reach each page
  // close together), they go through the caches non-temporally.
  const bool nontemporal = g.nontemporal != 0;  // uniform
  auto issue_block = [&](int pa, int slot0) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      int pid;
      const bool ok = page_ok(pa + u, pid);
      const uint8_t* rec = pool + (int64_t)(ok ? pid : 0) * page_bytes(D);
      if (nontemporal)
        dma_page<D, kCpolNonTemporal>(ring.ring[wv][slot0 + u], rec, lane);
      else
        dma_page<D>(ring.ring[wv][slot0 + u], rec, lane);
    }
  };
  const int nblk = (pend - pbeg + 1) >> 1;
  // RB-1 blocks ahead, issued unconditionally: a block past the wavefront's
  // pages loads page 0, unused.  Every block then costs the same number of
  // loads, so one constant wait count below finds the oldest block landed.
#pragma unroll
  for (int i = 0; i < RB - 1; ++i) issue_block(pbeg + 2 * i, 2 * i);
  lds_barrier();  // q operands visible to every wavefront; pages stay in flight
  QOps<D, QS, NRT> q;
#pragma unroll
  for (int n = 0; n < NRT; ++n) {
    q.crow[n] = sm.crow[16 * n + li];
    q.bias[n] = sm.qb[16 * n + li];
#pragma unroll
    for (int p = 0; p < QOps<D, QS, NRT>::NQ; ++p)
#pragma unroll
      for (int k = 0; k < QOps<D, QS, NRT>::STEPS; ++k) q.qf[n][p][k] = sm.qf[n][p][k][lane];
  }

  WaveState<D, NRT> st;
  st.init();
  // in groups of kRebiasBlocks blocks, the code bias taken out between groups
  for (int b0 = 0; b0 < nblk; b0 += kRebiasBlocks) {
    const int b1 = min(b0 + kRebiasBlocks, nblk);
    for (int b = b0; b < b1; ++b) {
      const int pa = pbeg + 2 * b;
      const int cs = 2 * (b % RB);
      // The compiler does not track global -> LDS loads: wait for them here.
      // In flight are blocks b .. b+RB-2 (issued in order): leave the younger
      // ones outstanding.
      __builtin_amdgcn_s_waitcnt(vmcnt_imm((RB - 2) * DMA_PER_BLOCK));
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (NK != NewKV::kNone) {
        if (b == b_cur)  // the one wavefront holding the current token (coded above)
          cur.put(ring.ring[wv][cs + (p_last - pa)], tok, lane);
      }
      PageRegs<D> c0, c1;
      lds_page<D>(c0, ring.ring[wv][cs], lane, lg);
      lds_page<D>(c1, ring.ring[wv][cs + 1], lane, lg);
      int pid0, pid1;
      const bool ok0 = page_ok(pa, pid0), ok1 = page_ok(pa + 1, pid1);
      // block b+RB-1 into the slots read one iteration ago; flies during compute.
      // With a 2-block ring every wait is vmcnt(0), so past the last block
      // nothing needs issuing; deeper rings keep the per-block count constant.
      if (RB > 2 || b + 1 < nblk) issue_block(pa + 2 * (RB - 1), 2 * ((b + RB - 1) % RB));
      attend_block_any<D, QS, NRT>(st, q, c0, c1, ok0, ok1, pa * kPageTokens, lo, hi, lg);
    }
    if (b1 < nblk) st.rebias();  // (the last group's bias comes out in finish())
  }

  st.finish();
  // ---- merge the W wavefronts: one LDS exchange ----
  // Every page load into this wavefront's ring has landed, so the wavefront
  // can dump its accumulators into its own ring without waiting for others.
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  f32x4* dump = reinterpret_cast<f32x4*>(&ring.ring[wv][0][0]);
#pragma unroll
  for (int n = 0; n < NRT; ++n) {
    const float lrow = row_sum4(st.l[n]);
    if (lg == 0) {
      sm.m[wv][16 * n + li] = st.m[n];
      sm.l[wv][16 * n + li] = lrow;
    }
#pragma unroll
    for (int t = 0; t < VT; ++t) dump[(n * VT + t) * 64 + lane] = st.acc[n][t];
  }
  if (lane == 0) sm.ev[wv] = st.ev;
  __syncthreads();
  // Wavefront wv merges output pairs wv, wv+W, ...: row 16n+li, channels
  // 16t+4lg .. +3.  Each wavefront's accumulators are relative to 2^m (its
  // running max) and carry P*sV scaled by 2^(kPvBias-ev).
  float Mr[PPW], Lr[PPW];
  f32x4 Ar[PPW];
#pragma unroll
  for (int k = 0; k < PPW; ++k) {
    const int pi = wv + k * W;
    Mr[k] = kNegInf;
    Lr[k] = 0.0f;
    Ar[k] = f32x4{0, 0, 0, 0};
    if (pi >= PAIRS) continue;  // wave-uniform
    const int row = 16 * (pi / VT) + li;
    float mm = kNegInf;
#pragma unroll
    for (int x = 0; x < W; ++x) mm = fmaxf(mm, sm.m[x][row]);
    const float mu = mm == kNegInf ? 0.0f : mm;
    float ll = 0.0f;
    f32x4 acc = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int x = 0; x < W; ++x) {
      const float e = fast_exp2(sm.m[x][row] - mu);
      ll += e * sm.l[x][row];
      const int evx = sm.ev[x];
      const float f = evx == kNoExp ? 0.0f : ldexp2(e, evx - kPvBias);
      acc += f * reinterpret_cast<const f32x4*>(&ring.ring[x][0][0])[pi * 64 + lane];
    }
    Mr[k] = mm;
    Lr[k] = ll;
    Ar[k] = acc;
  }

  if (nch == 1) {  // the workgroup saw the whole range: write the output
#pragma unroll
    for (int k = 0; k < PPW; ++k) {
      const int pi = wv + k * W;
      if (pi >= PAIRS) continue;
      const int row = 16 * (pi / VT) + li, t = pi % VT;
      if (row >= rb.nrows) continue;
      const float inv = Lr[k] > 0.0f ? 1.0f / Lr[k] : 0.0f;
      *reinterpret_cast<f32x4*>(out + (out_row0 + row) * D + 16 * t + 4 * lg) = Ar[k] * inv;
    }
    return;
  }

  // ---- several chunks: each wavefront publishes its pairs of the chunk's
  // record and counts its own arrival; for each wavefront index the last of
  // the chunks to arrive merges those pairs over all chunks.  No workgroup
  // barrier lies on this path. ----
  constexpr int64_t RS = ws_record_floats(D);
  constexpr int PF = kPairFloats;  // per pair: m[16], l[16], acc[4][64]
  const int64_t item = (int64_t)g.merge_begin + (int64_t)dw.rbl * a.batch + seq;
  const int64_t rec0 = (int64_t)g.ws_begin + ((int64_t)dw.rbl * a.batch + seq) * g.nchunk;
  if (wv >= PAIRS) return;  // (head_dim 64 with 16 rows: no pair for this wavefront)
  float* const recs = ws + kCounterWords;
  float* mine = recs + (rec0 + chunk) * RS;
#pragma unroll
  for (int k = 0; k < PPW; ++k) {
    const int pi = wv + k * W;
    if (pi >= PAIRS) continue;
    float* pr = mine + pi * PF;
    if (lg == 0) {
      st_dev(pr + li, Mr[k]);
      st_dev(pr + 16 + li, Lr[k]);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) st_dev(pr + 32 + e * 64 + lane, Ar[k][e]);
  }
  // the stores have completed before the arrival is counted
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  uint32_t* cnt = reinterpret_cast<uint32_t*>(ws) + (item * W + wv) * kCounterStride;
  uint32_t before = 0;
  if (lane == 0)
    before = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  before = __builtin_amdgcn_readfirstlane(before);
  if (before != (uint32_t)(nch - 1)) return;
  // the last arrival leaves the counter at zero for the next call
  if (lane == 0) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // ---- this wavefront's pairs over all chunks, folded in chunk order ----
  // (the order, not the arrival, fixes the rounding: results are deterministic)
  // Records are loaded only for chunks that exist, CB per round trip; this
  // wavefront's own chunk comes from its registers (the same values).  With
  // four pairs per wavefront, eight records per round trip would not fit the
  // registers.
  constexpr int CB = PPW >= 4 ? 4 : 8;
  float M[PPW], L[PPW];
  f32x4 A[PPW];
#pragma unroll
  for (int k = 0; k < PPW; ++k) {
    M[k] = kNegInf;
    L[k] = 0.0f;
    A[k] = f32x4{0, 0, 0, 0};
  }
  for (int c0 = 0; c0 < nch; c0 += CB) {
    float mc[PPW][CB], lc[PPW][CB];
    f32x4 ac[PPW][CB];
#pragma unroll
    for (int u = 0; u < CB; ++u) {
      const int c = c0 + u;
      if (c >= nch) break;  // wave-uniform
#pragma unroll
      for (int k = 0; k < PPW; ++k) {
        if (c == chunk) {
          mc[k][u] = Mr[k];
          lc[k][u] = Lr[k];
          ac[k][u] = Ar[k];
          continue;
        }
        const int pi = min(wv + k * W, PAIRS - 1);
        const float* r = recs + (rec0 + c) * RS + pi * PF;
        mc[k][u] = ld_dev(r + li);
        lc[k][u] = ld_dev(r + 16 + li);
#pragma unroll
        for (int e = 0; e < 4; ++e) ac[k][u][e] = ld_dev(r + 32 + e * 64 + lane);
      }
    }
#pragma unroll
    for (int u = 0; u < CB; ++u) {
      if (c0 + u >= nch) break;
#pragma unroll
      for (int k = 0; k < PPW; ++k) {
        const float mn = fmaxf(M[k], mc[k][u]);
        const float mu = mn == kNegInf ? 0.0f : mn;
        const float fa = fast_exp2(M[k] - mu), fb = fast_exp2(mc[k][u] - mu);
        L[k] = L[k] * fa + lc[k][u] * fb;
        A[k] = A[k] * fa + ac[k][u] * fb;
        M[k] = mn;
      }
    }
  }
#pragma unroll
  for (int k = 0; k < PPW; ++k) {
    const int pi = wv + k * W;
    if (pi >= PAIRS) continue;
    const int row = 16 * (pi / VT) + li, t = pi % VT;
    if (row >= rb.nrows) continue;
    const float inv = L[k] > 0.0f ? 1.0f / L[k] : 0.0f;
    *reinterpret_cast<f32x4*>(out + (out_row0 + row) * D + 16 * t + 4 * lg) = A[k] * inv;
  }
}

// ---------------------------------------------------------------------------
// Append: one workgroup = W consecutive tokens of one (layer, sequence, row
// block), one wavefront per token carrying that token's heads.  The tokens'
// key ranges nearly coincide, so the workgroup streams the union of their
// pages HBM -> LDS once, through a ring of RB two-page blocks shared by all
// wavefronts: each block's 1 KiB pieces and scale blocks are spread over the
// wavefronts, and one barrier per block both publishes a landed block and
// frees the slot the next load reuses.  Each wavefront masks the keys to its
// own token's causal (and window) range.
// ---------------------------------------------------------------------------
template <int D>
struct AppendGeo {
  static constexpr int KIB = 32 * D / 1024;        // 1 KiB code pieces per page
  static constexpr int PIECES = 2 * KIB + 2;       // per block: code pieces + two scale blocks
};

template <int D, int W, int RB>
struct alignas(16) AppendLds {
  uint8_t ring[RB][2][lds_slot_bytes<D>()];
  int ok[RB][2];  // page of the slot exists (in range, id inside the pool)
};

template <int D, int QS, int NRT>
__global__ __launch_bounds__(kAppendWaves * 64) void append_kernel(
    const AppendArgs a, const void* __restrict__ qp, float* __restrict__ out,
    const uint8_t* __restrict__ pool, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ context_lens, const int32_t* __restrict__ cu_q_lens) {
  constexpr int W = kAppendWaves, RB = kAppendRing;
  constexpr int VT = Geo<D>::VT;
  constexpr int KIB = AppendGeo<D>::KIB, PIECES = AppendGeo<D>::PIECES;
  constexpr int MY_PIECES_MAX = (PIECES + W - 1) / W;
  __shared__ AppendLds<D, W, RB> sm;
  const int w = swizzled_block(a.total_wgs);
  if (w >= a.total_wgs) return;
  uint32_t q_, r_;
  udiv_recip((uint32_t)w, (uint32_t)a.token_blocks, a.tb_recip, q_, r_);
  const int tb = (int)r_;
  udiv_recip(q_, (uint32_t)a.head_blocks, a.hb_recip, q_, r_);
  const int hb = (int)r_;
  // layers are enumerated innermost after the sequence so that the layers
  // sharing a slot (adjacent in a.order) read the same pages back to back
  udiv_recip(q_, (uint32_t)a.num_layers, a.layer_recip, q_, r_);
  const int oi = (int)r_;
  const int seq = (int)q_;
  const AppendArgs* ka = first_kernel_arg<AppendArgs>();
  const int layer = ka->order[oi];
  const int slot = ka->layer_slot[layer];
  const int window = ka->layer_window[layer];

  const int lane = lane_id(), li = lane & 15, lg = lane >> 4;
  const int wv = threadIdx.x >> 6;
  const int q0 = cu_q_lens[seq];
  const int qlen = cu_q_lens[seq + 1] - q0;
  const int t0 = tb * W;
  if (t0 >= qlen || q0 < 0 || q0 + qlen > a.total_q) return;  // workgroup-uniform
  const int nt = min(W, qlen - t0);                            // tokens of this workgroup
  const int ctx = clamp_ctx(context_lens[seq], a.max_context, a.max_pages);
  const int t = t0 + wv;
  const bool live = wv < nt;
  // this wavefront's position; a wavefront past the chunk's last token runs
  // that token's key range (valid data, no branch around the attention) and
  // writes nothing
  const int p = ctx - qlen + min(t, t0 + nt - 1);
  const int head0 = hb * kRowsPerBlock;
  const int nrows = min(kRowsPerBlock, a.num_q_heads - head0);
  const int64_t row0 = ((int64_t)layer * a.total_q + q0 + min(t, qlen - 1)) * a.num_q_heads + head0;

  // the union of the tokens' key ranges
  const int p_lo = ctx - qlen + t0, p_hi = ctx - qlen + t0 + nt - 1;
  const int lo_u = window > 0 ? max(0, p_lo - window + 1) : 0;
  const int hi_u = p_hi + 1;
  if (hi_u <= 0 || lo_u >= hi_u) {  // no key at all (context shorter than the chunk)
    if (live)
      for (int n = 0; n < NRT; ++n) {
        const int row = 16 * n + li;
        if (row < nrows)
          for (int tt = 0; tt < VT; ++tt)
            *reinterpret_cast<f32x4*>(out + (row0 + row) * D + 16 * tt + 4 * lg) =
                f32x4{0, 0, 0, 0};
      }
    return;
  }
  const int pbeg = lo_u >> 4, pend = ((hi_u - 1) >> 4) + 1;
  const int nblk = (pend - pbeg + 1) >> 1;
  // this wavefront's own key range (positions below 0 have no keys)
  const int hi = p + 1;
  const int lo = window > 0 ? max(0, p - window + 1) : 0;

  // q first (converted before any page load is issued, so that its wait does
  // not also wait for pages)
  constexpr int esz = QS == 1 ? 2 : 4;
  QRaw<D, QS, NRT> qr;
  load_q_raw<D, QS, NRT>(qr, static_cast<const uint8_t*>(qp) + row0 * D * esz, nrows, li, lg);
  QOps<D, QS, NRT> q;
  convert_q<D, QS, NRT>(q, qr, a.scale_log2, nrows, li);
  __builtin_amdgcn_sched_barrier(0);

  // page ids, a window of 64 per register, reloaded when the loads pass it
  const int32_t* table_row = block_table + ((int64_t)slot * a.batch + seq) * (int64_t)a.max_pages;
  int wbase = pbeg;
  int ids = pbeg + lane < pend ? table_row[pbeg + lane] : -1;
  // this wavefront's share of block `blk`'s loads into ring slot `rs` (the
  // wavefront index read as uniform, so that the page checks are scalar)
  const int wvs = __builtin_amdgcn_readfirstlane(wv);
  const uint32_t pool_pages = (uint32_t)min<int64_t>(a.num_pages, 0xFFFFFFFF);
  auto issue_block = [&](int blk, int rs) {
#pragma unroll
    for (int i = 0; i < MY_PIECES_MAX; ++i) {
      const int k = wvs + i * W;
      if (k >= PIECES) break;  // wave-uniform
      const int u = k < 2 * KIB ? k / KIB : k - 2 * KIB;
      const int pg = pbeg + 2 * blk + u;
      if (pg - wbase >= 64) {  // wave-uniform
        wbase = pg;
        ids = pg + lane < pend ? table_row[pg + lane] : -1;
      }
      const int pid = __builtin_amdgcn_readlane(ids, min(max(pg - wbase, 0), 63));
      const bool ok = pg < pend && (uint32_t)pid < pool_pages;
      const uint8_t* rec = pool + (int64_t)(ok ? pid : 0) * page_bytes(D);
      uint8_t* dst = sm.ring[rs][u];
      if (k < 2 * KIB) {
        const int h = k % KIB;
        __builtin_amdgcn_global_load_lds(rec + h * 1024 + lane * 16, dst + h * 1024, 16, 0, 0);
        if (h == 0 && lane == 0) sm.ok[rs][u] = ok;
      } else {
        __builtin_amdgcn_global_load_lds(rec + 32 * D + 4 * min(lane, 31), dst + 32 * D, 4, 0, 0);
      }
    }
  };
  // loads per block issued by this wavefront (constant: every block issues
  // all its pieces; blocks past the range load page 0, unused)
  const int mine = (PIECES - wvs + W - 1) / W;
#pragma unroll
  for (int i = 0; i < RB - 1; ++i) issue_block(i, i);

  WaveState<D, NRT> st;
  st.init();
  for (int b = 0; b < nblk; ++b) {
    const int rs = b % RB;
    if (b % kRebiasBlocks == 0 && b > 0) st.rebias();  // the code bias out (wave-uniform)
    // this wavefront's pieces of block b have landed (blocks b+1 .. b+RB-2
    // may still be in flight) ...
    // (a page-id reload among the younger loads only makes this wait longer)
    static_assert(MY_PIECES_MAX <= 2, "wait counts below");
    if (mine == 2) {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm((RB - 2) * 2));
    } else if (mine == 1) {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm((RB - 2) * 1));
    }
    // ... and, past the barrier, every wavefront's; every wavefront is also
    // done with the slot that block b+RB-1 now reuses
    lds_barrier();
    issue_block(b + RB - 1, (b + RB - 1) % RB);
    PageRegs<D> c0, c1;
    lds_page<D>(c0, sm.ring[rs][0], lane, lg);
    lds_page<D>(c1, sm.ring[rs][1], lane, lg);
    const int pos0 = (pbeg + 2 * b) * kPageTokens;
    attend_block_any<D, QS, NRT>(st, q, c0, c1, sm.ok[rs][0] != 0, sm.ok[rs][1] != 0, pos0, lo, hi,
                                 lg);
  }
  // every load of this wavefront has landed before the workgroup exits
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  if (!live) return;
  st.finish();
#pragma unroll
  for (int n = 0; n < NRT; ++n) {
    const int row = 16 * n + li;
    const float l = row_sum4(st.l[n]);
    if (row >= nrows) continue;
    const float inv = (l > 0.0f && st.ev != kNoExp) ? ldexp2(1.0f / l, st.ev - kPvBias) : 0.0f;
    float* o = out + (row0 + row) * D + 4 * lg;
#pragma unroll
    for (int tt = 0; tt < VT; ++tt) *reinterpret_cast<f32x4*>(o + 16 * tt) = st.acc[n][tt] * inv;
  }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
static inline dim3 padded_grid(int total) { return dim3((unsigned)((total + 7) / 8 * 8)); }

template <int D, int QS, int NRT, NewKV NK, int W>
static hipError_t launch_decode_t(const DecodeArgs& a, const DecodePtrs& p, hipStream_t stream) {
  hipLaunchKernelGGL((decode_kernel<D, QS, NRT, NK, W>), padded_grid(a.total_wgs), dim3(W * 64), 0,
                     stream, a, p.q, p.out, p.pool, p.block_table, p.context_lens, p.ws, p.k_new,
                     p.v_new);
  return hipGetLastError();
}

template <int D, int QS, int NRT, int W>
static hipError_t launch_decode_w(NewKV nk, const DecodeArgs& a, const DecodePtrs& p,
                                  hipStream_t stream) {
  if (nk == NewKV::kBf16) return launch_decode_t<D, QS, NRT, NewKV::kBf16, W>(a, p, stream);
  if (nk == NewKV::kF32) return launch_decode_t<D, QS, NRT, NewKV::kF32, W>(a, p, stream);
  return launch_decode_t<D, QS, NRT, NewKV::kNone, W>(a, p, stream);
}

template <int D, int QS, int NRT>
static hipError_t launch_decode_n(int waves, NewKV nk, const DecodeArgs& a, const DecodePtrs& p,
                                  hipStream_t stream) {
  if (waves == kDecodeWavesSmall) return launch_decode_w<D, QS, NRT, kDecodeWavesSmall>(nk, a, p, stream);
  return launch_decode_w<D, QS, NRT, kDecodeWaves>(nk, a, p, stream);
}

hipError_t launch_decode(int D, bool q_f32, int nrt, int waves, NewKV nk, const DecodeArgs& a,
                         const DecodePtrs& p, hipStream_t stream) {
#define MQA_DEC(DD, QQ, NN) return launch_decode_n<DD, QQ, NN>(waves, nk, a, p, stream)
  // fp32 queries run one 16-row tile per wavefront (the planner's rows)
  if (q_f32 && nrt != 1) return hipErrorInvalidValue;
  if (D == 128) {
    if (q_f32) MQA_DEC(128, 2, 1);
    if (nrt == 1) MQA_DEC(128, 1, 1);
    MQA_DEC(128, 1, 2);
  }
  if (q_f32) MQA_DEC(64, 2, 1);
  if (nrt == 1) MQA_DEC(64, 1, 1);
  MQA_DEC(64, 1, 2);
#undef MQA_DEC
}

template <int D, int QS, int NRT>
static hipError_t launch_append_t(const AppendArgs& a, const AppendPtrs& p, hipStream_t stream) {
  hipLaunchKernelGGL((append_kernel<D, QS, NRT>), padded_grid(a.total_wgs), dim3(kAppendWaves * 64),
                     0, stream, a, p.q, p.out, p.pool, p.block_table, p.context_lens, p.cu_q_lens);
  return hipGetLastError();
}

hipError_t launch_append(int D, bool q_f32, int nrt, const AppendArgs& a, const AppendPtrs& p,
                         hipStream_t stream) {
#define MQA_APP(DD, QQ, NN) return launch_append_t<DD, QQ, NN>(a, p, stream)
  if (D == 128) {
    if (q_f32) { if (nrt == 1) MQA_APP(128, 2, 1); MQA_APP(128, 2, 2); }
    if (nrt == 1) MQA_APP(128, 1, 1);
    MQA_APP(128, 1, 2);
  }
  if (q_f32) { if (nrt == 1) MQA_APP(64, 2, 1); MQA_APP(64, 2, 2); }
  if (nrt == 1) MQA_APP(64, 1, 1);
  MQA_APP(64, 1, 2);
#undef MQA_APP
}

}  // namespace mqa
