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
//  * Keys are processed two pages (32 keys) at a time.  Page bytes arrive
//    with one 16-byte load per lane per 1 KiB (layout.hpp) and are turned
//    into exact fp16 integers in registers.
//  * S^T = K.Q^T and O^T += V^T.P^T run on 16x16x32 fp16 matrix cores with
//    fp32 accumulation.  The S^T tile a lane receives (4 keys of one row) is
//    exactly the P^T operand it needs, so the softmax stays in registers.
//  * q is scaled per row by a power of two so that its largest element lies
//    in [2^14, 2^15): bf16 q is then exact in fp16; fp32 q is split into two
//    fp16 terms.  P*sV is scaled by a power of two tied to the largest V scale
//    seen so far, so the fp16 P operand keeps full precision.  The int8
//    codes, the products and the fp32 sums make the only roundings the fp16
//    P operand (relative 2^-11) and fp32 accumulation.
//  * Online softmax in the log2 domain (v_exp_f32), with max and sum per row.
//  * Decode splits long contexts into chunks (flash-decoding style): the
//    wavefronts of a workgroup take consecutive pages and are merged through
//    LDS; chunks of one sequence are merged by merge_kernel.
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
template <int D, int QS, int NRT>
struct QOps {
  f16x8 q[NRT][QS][Geo<D>::KSTEPS];
  float crow[NRT];  // 2^(E-15) * scale * log2(e): undoes the row's prescale
};

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

// Turn the raw rows into matrix-core operands: scale each row by a power of
// two so that its largest |element| lies in [2^14, 2^15), then round to fp16
// (exact for bf16 input; fp32 input becomes a sum of two fp16 terms).
template <int D, int QS, int NRT>
__device__ __forceinline__ void convert_q(QOps<D, QS, NRT>& o, const QRaw<D, QS, NRT>& r,
                                          float scale_log2, int nrows, int li) {
  constexpr int CH = Geo<D>::CH;
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
    a = row_max4(a);
    const int E = a > 0.0f ? max(frexp_exp(a), -100) : 15;
    const float sc = ldexp2(1.0f, 15 - E);
    o.crow[n] = ldexp2(scale_log2, E - 15);
#pragma unroll
    for (int s = 0; s < Geo<D>::KSTEPS; ++s) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float y = x[8 * s + e] * sc;
        const _Float16 h1 = (_Float16)y;
        o.q[n][0][s][e] = h1;
        if constexpr (QS == 2) o.q[n][1][s][e] = (_Float16)(y - (float)h1);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// One wavefront's running softmax state over its keys
// ---------------------------------------------------------------------------
template <int D, int NRT>
struct WaveState {
  f32x4 acc[NRT][Geo<D>::VT];  // O^T tiles: lane (i, g) holds channels 16t+4g..+3 of row i
  float m[NRT];                // running max (log2 domain), equal on a row's 4 lanes
  float l[NRT];                // this lane's part of the row's running sum
  int ev;                      // exponent of the largest V scale seen (kNoExp: none)

  __device__ __forceinline__ void init() {
#pragma unroll
    for (int n = 0; n < NRT; ++n) {
      m[n] = kNegInf;
      l[n] = 0.0f;
#pragma unroll
      for (int t = 0; t < Geo<D>::VT; ++t) acc[n][t] = f32x4{0, 0, 0, 0};
    }
    ev = kNoExp;
  }
};

// Attend the 32 keys of two consecutive logical pages.  pos0 is the position
// of the first page's first token; keys outside [lo, hi) or on a page that is
// not ok are masked (their bytes are never used, so poison is harmless).
template <int D, int QS, int NRT>
__device__ __forceinline__ void attend_block(WaveState<D, NRT>& st, const QOps<D, QS, NRT>& q,
                                             const PageRegs<D>& p0, const PageRegs<D>& p1,
                                             bool masked, bool ok0, bool ok1, int pos0, int lo,
                                             int hi, int lg) {
  constexpr int KS = Geo<D>::KSTEPS;
  // S^T for both pages: lane (i, g) gets the scores of keys 4g..4g+3 for row i.
  f32x4 s[NRT][2];
#pragma unroll
  for (int n = 0; n < NRT; ++n) s[n][0] = s[n][1] = f32x4{0, 0, 0, 0};
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const PageRegs<D>& P = u ? p1 : p0;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int h = ks >> 1, dw = (ks & 1) * 2;
      const f16x8 kop = i8x8_to_f16x8(P.k[h][dw], P.k[h][dw + 1]);
#pragma unroll
      for (int n = 0; n < NRT; ++n)
#pragma unroll
        for (int qs = 0; qs < QS; ++qs) s[n][u] = mma16(kop, q.q[n][qs][ks], s[n][u]);
    }
  }

  bool valid[2][4];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int pos = pos0 + 16 * u + 4 * lg + r;
      valid[u][r] = !masked || ((u ? ok1 : ok0) && pos >= lo && pos < hi);
    }

  // Largest valid V scale of the block -> running exponent (wave-uniform).
  float vmax = 0.0f;
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (valid[u][r]) vmax = fmaxf(vmax, (u ? p1.sv : p0.sv)[r]);
  vmax = row_max4(vmax);
  int ev_new = st.ev;
  // (clamped so that 2^(14-ev) stays finite for absurdly small scales)
  if (vmax > 0.0f) ev_new = max(ev_new, max(frexp_exp(vmax), -100));
  const int dexp = st.ev == kNoExp ? 0 : st.ev - ev_new;
  st.ev = ev_new;
  const float pvm = ev_new == kNoExp ? 0.0f : ldexp2(1.0f, 14 - ev_new);

  f16x8 pop[NRT];
#pragma unroll
  for (int n = 0; n < NRT; ++n) {
    float sig[2][4];
    float mx = kNegInf;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float sk = (u ? p1.sk : p0.sk)[r];
        sig[u][r] = valid[u][r] ? s[n][u][r] * (sk * q.crow[n]) : kNegInf;
        mx = fmaxf(mx, sig[u][r]);
      }
    mx = row_max4(mx);
    const float m_new = fmaxf(st.m[n], mx);
    const float m_use = m_new == kNegInf ? 0.0f : m_new;
    const float alpha = fast_exp2(st.m[n] - m_use);
    float ps = 0.0f;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = fast_exp2(sig[u][r] - m_use);
        ps += p;
        const float pv = valid[u][r] ? p * ((u ? p1.sv : p0.sv)[r] * pvm) : 0.0f;
        pop[n][4 * u + r] = (_Float16)pv;
      }
    st.l[n] = st.l[n] * alpha + ps;
    st.m[n] = m_new;
    const float ascale = ldexp2(alpha, dexp);
#pragma unroll
    for (int t = 0; t < Geo<D>::VT; ++t) st.acc[n][t] *= ascale;
  }

#pragma unroll
  for (int t = 0; t < Geo<D>::VT; ++t) {
    const int h = t >> 2, dw = t & 3;
    f16x2 a0, a1, b0, b1;
    i8x4_to_f16x4(p0.v[h][dw], a0, a1);
    i8x4_to_f16x4(p1.v[h][dw], b0, b1);
    const f16x8 vop = {a0[0], a0[1], a1[0], a1[1], b0[0], b0[1], b1[0], b1[1]};
#pragma unroll
    for (int n = 0; n < NRT; ++n) st.acc[n][t] = mma16(vop, pop[n], st.acc[n][t]);
  }
}

// Logical pages [pbeg, pend) of one (slot, sequence), read two at a time.
// The wavefront keeps a window of 64 page ids in a register (lane i holds the
// id of page wbase + i), filled by one coalesced load and handed out with
// readlane, so the page loads never wait on a table read of their own.
template <int D>
struct PageStream {
  const uint8_t* __restrict__ pool;
  const int32_t* __restrict__ table_row;
  int64_t num_pages;
  int pend;
  int lane, lg;
  int ids, wbase;
  PageRegs<D> c0, c1;
  bool ok0, ok1;

  __device__ __forceinline__ void load_ids(int from) {
    wbase = from;
    ids = from + lane < pend ? table_row[from + lane] : -1;
  }
  // Branch-free: a page outside [.., pend) or with an id outside the pool
  // loads page 0 instead (it exists: num_pages >= 1) and is masked by ok.
  template <bool RELOAD>
  __device__ __forceinline__ void fetch(PageRegs<D>& r, int pi, bool& ok) {
    if constexpr (RELOAD) {
      if (pi - wbase >= 64) load_ids(pi);
    }
    const int pid = __builtin_amdgcn_readlane(ids, min(pi - wbase, 63));
    ok = pi < pend && (uint32_t)pid < (uint64_t)num_pages;
    load_page<D>(r, pool + (int64_t)(ok ? pid : 0) * page_bytes(D), lane, lg);
  }
  // issue the first pair's loads
  template <bool RELOAD>
  __device__ __forceinline__ void start(int pbeg) {
    fetch<RELOAD>(c0, pbeg, ok0);
    fetch<RELOAD>(c1, pbeg + 1, ok1);
  }
};

// Attend pages [pbeg, ps.pend) whose first pair ps.start(pbeg) already issued;
// the next pair's loads are issued before the current pair is computed.
template <int D, int QS, int NRT, bool RELOAD>
__device__ __forceinline__ void attend_pages(WaveState<D, NRT>& st, const QOps<D, QS, NRT>& q,
                                             PageStream<D>& ps, int pbeg, int lo, int hi) {
  for (int pa = pbeg; pa < ps.pend; pa += 2) {
    PageRegs<D> n0, n1;
    bool nok0 = false, nok1 = false;
    const bool more = pa + 2 < ps.pend;
    if (more) {
      ps.template fetch<RELOAD>(n0, pa + 2, nok0);
      ps.template fetch<RELOAD>(n1, pa + 3, nok1);
    }
    const int pos0 = pa * kPageTokens;
    const bool masked = !(ps.ok0 && ps.ok1 && pos0 >= lo && pos0 + 2 * kPageTokens <= hi);
    attend_block<D, QS, NRT>(st, q, ps.c0, ps.c1, masked, ps.ok0, ps.ok1, pos0, lo, hi, ps.lg);
    if (more) {
      ps.c0 = n0;
      ps.c1 = n1;
      ps.ok0 = nok0;
      ps.ok1 = nok1;
    }
  }
}

__device__ __forceinline__ int clamp_ctx(int ctx, int max_context, int max_pages) {
  const int cap = min(max_context, max_pages * kPageTokens);
  return min(max(ctx, 0), cap);
}

// Chunk count of a decode sequence: pages of [lo, hi) split ppc per chunk.
__device__ __forceinline__ void decode_range(int ctx, int window, int& lo, int& hi) {
  hi = ctx;
  lo = window > 0 ? max(0, ctx - window) : 0;
}

// XCD-aware flat index: hardware workgroup x runs on XCD x % 8, so give each
// XCD a contiguous range of logical work (gridDim.x is a multiple of 8).
__device__ __forceinline__ int swizzled_block() {
  const int nx = gridDim.x, x = blockIdx.x;
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

__device__ __forceinline__ DecodeWork decode_work(const DecodeArgs& a, int w) {
  int gi = 0;
  while (gi + 1 < a.num_groups && w >= a.groups[gi + 1].wg_begin) ++gi;
  DecodeWork d;
  d.g = a.groups[gi];
  int local = w - d.g.wg_begin;
  d.rbl = local % d.g.num_rb;
  local /= d.g.num_rb;
  d.chunk = local % d.g.nchunk;
  d.seq = local / d.g.nchunk;
  d.rb = a.rbs[d.g.first_rb + d.rbl];
  return d;
}

// Merge the nch partial records of one (row block, sequence) into the output.
// 256 threads: thread t takes row t/8 and D/8 consecutive channels.
template <int D>
__device__ __forceinline__ void merge_records(const float* __restrict__ rec0, int nch, int nrows,
                                              float* __restrict__ out_rows) {
  const int row = threadIdx.x >> 3, part = threadIdx.x & 7;
  if (row >= nrows) return;
  constexpr int PER = D / 8;
  constexpr int64_t RS = ws_record_floats(D);
  float mm = kNegInf;
  for (int c = 0; c < nch; ++c) mm = fmaxf(mm, rec0[c * RS + row]);
  const float mu = mm == kNegInf ? 0.0f : mm;
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.0f;
  float ll = 0.0f;
  for (int c = 0; c < nch; ++c) {
    const float* rec = rec0 + c * RS;
    const float f = fast_exp2(rec[row] - mu);
    ll += f * rec[32 + row];
    const float* src = rec + 64 + row * D + part * PER;
#pragma unroll
    for (int e = 0; e < PER; e += 4) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(src + e);
      acc[e] += f * x[0];
      acc[e + 1] += f * x[1];
      acc[e + 2] += f * x[2];
      acc[e + 3] += f * x[3];
    }
  }
  const float inv = ll > 0.0f ? 1.0f / ll : 0.0f;
  float* o = out_rows + row * D + part * PER;
#pragma unroll
  for (int e = 0; e < PER; e += 4)
    *reinterpret_cast<f32x4*>(o + e) =
        f32x4{acc[e] * inv, acc[e + 1] * inv, acc[e + 2] * inv, acc[e + 3] * inv};
}

template <int D, int QS, int NRT>
__global__ __launch_bounds__(kAttnWaves * 64) void decode_kernel(
    const DecodeArgs a, const void* __restrict__ qp, float* __restrict__ out,
    const uint8_t* __restrict__ pool, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ context_lens, float* __restrict__ ws,
    uint32_t* __restrict__ counters) {
  constexpr int VT = Geo<D>::VT;
  const int w = swizzled_block();
  if (w >= a.total_wgs) return;
  const DecodeWork dw = decode_work(a, w);
  const DecodeGroup& g = dw.g;
  const RowBlock& rb = dw.rb;
  const int seq = dw.seq, chunk = dw.chunk;

  const int lane = lane_id(), li = lane & 15, lg = lane >> 4;
  const int wv = threadIdx.x >> 6;
  const int ctx = clamp_ctx(context_lens[seq], a.max_context, a.max_pages);
  int lo, hi;
  decode_range(ctx, g.window, lo, hi);
  const int64_t out_row0 = ((int64_t)rb.layer * a.batch + seq) * a.num_q_heads + rb.head0;

  if (hi <= lo) {  // empty context: zeros
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
  const int p_first = lo >> 4, p_last = (hi - 1) >> 4;
  const int ppc = g.pages_per_wave * kAttnWaves;
  const int nch = (p_last - p_first + ppc) / ppc;
  if (chunk >= nch) return;

  // q loads first, then this wavefront's first page pair, then convert q
  // while the pages are in flight.
  // Order of the memory traffic: this wavefront's page ids, its query rows,
  // its first page pair (once the ids are in); q is converted while the
  // pages are in flight.
  const int pbeg = p_first + chunk * ppc + wv * g.pages_per_wave;
  PageStream<D> ps;
  ps.pool = pool;
  ps.table_row = block_table + ((int64_t)g.slot * a.batch + seq) * (int64_t)a.max_pages;
  ps.num_pages = a.num_pages;
  ps.pend = min(pbeg + g.pages_per_wave, p_last + 1);
  ps.lane = lane;
  ps.lg = lg;
  ps.load_ids(pbeg);
  constexpr int esz = QS == 1 ? 2 : 4;
  QRaw<D, QS, NRT> qr;
  load_q_raw<D, QS, NRT>(qr, static_cast<const uint8_t*>(qp) + out_row0 * D * esz, rb.nrows, li,
                         lg);
  ps.template start<false>(pbeg);  // branch-free: pages past pend load page 0, masked
  // keep the page loads issued ahead of the q conversion
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  QOps<D, QS, NRT> q;
  convert_q<D, QS, NRT>(q, qr, a.scale_log2, rb.nrows, li);

  WaveState<D, NRT> st;
  st.init();
  attend_pages<D, QS, NRT, false>(st, q, ps, pbeg, lo, hi);

  // ---- merge the wavefronts of the workgroup through LDS ----
  __shared__ float sm_m[kAttnWaves][32];
  __shared__ float sm_l[kAttnWaves][32];
  __shared__ f32x4 sm_acc[kAttnWaves - 1][NRT][VT][64];
  __shared__ int sm_last;
#pragma unroll
  for (int n = 0; n < NRT; ++n) {
    const float lrow = row_sum4(st.l[n]);
    if (lg == 0) {
      sm_m[wv][16 * n + li] = st.m[n];
      sm_l[wv][16 * n + li] = lrow;
    }
  }
  __syncthreads();
  float M[NRT], L[NRT];
#pragma unroll
  for (int n = 0; n < NRT; ++n) {
    const int row = 16 * n + li;
    float mm = kNegInf;
#pragma unroll
    for (int x = 0; x < kAttnWaves; ++x) mm = fmaxf(mm, sm_m[x][row]);
    const float mu = mm == kNegInf ? 0.0f : mm;
    float ll = 0.0f;
#pragma unroll
    for (int x = 0; x < kAttnWaves; ++x) ll += fast_exp2(sm_m[x][row] - mu) * sm_l[x][row];
    M[n] = mm;
    L[n] = ll;
    const float fac = st.ev == kNoExp ? 0.0f : ldexp2(fast_exp2(st.m[n] - mu), st.ev - 14);
#pragma unroll
    for (int t = 0; t < VT; ++t) st.acc[n][t] *= fac;
  }
  if (wv > 0) {
#pragma unroll
    for (int n = 0; n < NRT; ++n)
#pragma unroll
      for (int t = 0; t < VT; ++t) sm_acc[wv - 1][n][t][lane] = st.acc[n][t];
  }
  __syncthreads();
  if (wv == 0) {
#pragma unroll
    for (int x = 1; x < kAttnWaves; ++x)
#pragma unroll
      for (int n = 0; n < NRT; ++n)
#pragma unroll
        for (int t = 0; t < VT; ++t) st.acc[n][t] += sm_acc[x - 1][n][t][lane];
  }

  if (nch == 1) {  // the workgroup saw the whole range: write the output
    if (wv != 0) return;
#pragma unroll
    for (int n = 0; n < NRT; ++n) {
      const int row = 16 * n + li;
      if (row >= rb.nrows) continue;
      const float inv = L[n] > 0.0f ? 1.0f / L[n] : 0.0f;
      float* o = out + (out_row0 + row) * D + 4 * lg;
#pragma unroll
      for (int t = 0; t < VT; ++t) *reinterpret_cast<f32x4*>(o + 16 * t) = st.acc[n][t] * inv;
    }
    return;
  }

  // ---- several chunks: publish this chunk's partial; the last chunk of the
  // (row block, sequence) to arrive merges them all ----
  const int64_t mi = (int64_t)g.merge_begin + (int64_t)dw.rbl * a.batch + seq;
  float* rec0 =
      ws + ((int64_t)g.ws_begin + ((int64_t)dw.rbl * a.batch + seq) * g.nchunk) * ws_record_floats(D);
  if (wv == 0) {
    float* rec = rec0 + (int64_t)chunk * ws_record_floats(D);
#pragma unroll
    for (int n = 0; n < NRT; ++n) {
      const int row = 16 * n + li;
      if (lg == 0) {
        rec[row] = M[n];
        rec[32 + row] = L[n];
      }
      float* o = rec + 64 + row * D + 4 * lg;
#pragma unroll
      for (int t = 0; t < VT; ++t) *reinterpret_cast<f32x4*>(o + 16 * t) = st.acc[n][t];
    }
  }
  __threadfence();  // release: the record is visible to every XCD before the count
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev = atomicAdd(counters + mi, 1u);
    sm_last = prev == (uint32_t)(nch - 1);
  }
  __syncthreads();
  if (!sm_last) return;
  __threadfence();  // acquire: see every other chunk's record
  merge_records<D>(rec0, nch, rb.nrows, out + out_row0 * D);
  if (threadIdx.x == 0) atomicExch(counters + mi, 0u);  // ready for the next call
}

// ---------------------------------------------------------------------------
// Append: one wavefront = all heads of a row block for one chunk token; the
// workgroup's four wavefronts take four consecutive tokens (their key ranges
// nearly coincide, so their page reads hit the same cache lines).
// ---------------------------------------------------------------------------
template <int D, int QS, int NRT>
__global__ __launch_bounds__(kAttnWaves * 64) void append_kernel(
    const AppendArgs a, const void* __restrict__ qp, float* __restrict__ out,
    const uint8_t* __restrict__ pool, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ context_lens, const int32_t* __restrict__ cu_q_lens) {
  constexpr int VT = Geo<D>::VT;
  const int w = swizzled_block();
  if (w >= a.total_wgs) return;
  int local = w;
  const int tb = local % a.token_blocks;
  local /= a.token_blocks;
  const int hb = local % a.head_blocks;
  local /= a.head_blocks;
  // layers are enumerated innermost after the sequence so that the layers
  // sharing a slot (adjacent in a.order) read the same pages back to back
  const int oi = local % a.num_layers;
  const int seq = local / a.num_layers;
  const int layer = a.order[oi];
  const int slot = a.layer_slot[layer];
  const int window = a.layer_window[layer];

  const int lane = lane_id(), li = lane & 15, lg = lane >> 4;
  const int wv = threadIdx.x >> 6;
  const int q0 = cu_q_lens[seq];
  const int qlen = cu_q_lens[seq + 1] - q0;
  const int t = tb * kAttnWaves + wv;
  if (t >= qlen || q0 < 0 || q0 + t >= a.total_q) return;
  const int ctx = clamp_ctx(context_lens[seq], a.max_context, a.max_pages);
  const int p = ctx - qlen + t;
  const int head0 = hb * kRowsPerBlock;
  const int nrows = min(kRowsPerBlock, a.num_q_heads - head0);
  const int64_t row0 = ((int64_t)layer * a.total_q + q0 + t) * a.num_q_heads + head0;
  if (p < 0) {
    for (int n = 0; n < NRT; ++n) {
      const int row = 16 * n + li;
      if (row < nrows)
        for (int tt = 0; tt < VT; ++tt)
          *reinterpret_cast<f32x4*>(out + (row0 + row) * D + 16 * tt + 4 * lg) =
              f32x4{0, 0, 0, 0};
    }
    return;
  }
  const int hi = p + 1;
  const int lo = window > 0 ? max(0, p - window + 1) : 0;

  constexpr int esz = QS == 1 ? 2 : 4;
  QRaw<D, QS, NRT> qr;
  load_q_raw<D, QS, NRT>(qr, static_cast<const uint8_t*>(qp) + row0 * D * esz, nrows, li, lg);
  const int pbeg = lo >> 4;
  PageStream<D> ps;
  ps.pool = pool;
  ps.table_row = block_table + ((int64_t)slot * a.batch + seq) * (int64_t)a.max_pages;
  ps.num_pages = a.num_pages;
  ps.pend = ((hi - 1) >> 4) + 1;
  ps.lane = lane;
  ps.lg = lg;
  ps.load_ids(pbeg);
  ps.template start<true>(pbeg);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  QOps<D, QS, NRT> q;
  convert_q<D, QS, NRT>(q, qr, a.scale_log2, nrows, li);
  WaveState<D, NRT> st;
  st.init();
  attend_pages<D, QS, NRT, true>(st, q, ps, pbeg, lo, hi);
#pragma unroll
  for (int n = 0; n < NRT; ++n) {
    const int row = 16 * n + li;
    const float l = row_sum4(st.l[n]);
    if (row >= nrows) continue;
    const float inv = (l > 0.0f && st.ev != kNoExp) ? ldexp2(1.0f / l, st.ev - 14) : 0.0f;
    float* o = out + (row0 + row) * D + 4 * lg;
#pragma unroll
    for (int tt = 0; tt < VT; ++tt) *reinterpret_cast<f32x4*>(o + 16 * tt) = st.acc[n][tt] * inv;
  }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
static inline dim3 padded_grid(int total) { return dim3((unsigned)((total + 7) / 8 * 8)); }

template <int D, int QS, int NRT>
static hipError_t launch_decode_t(const DecodeArgs& a, const DecodePtrs& p, hipStream_t stream) {
  hipLaunchKernelGGL((decode_kernel<D, QS, NRT>), padded_grid(a.total_wgs), dim3(kAttnWaves * 64),
                     0, stream, a, p.q, p.out, p.pool, p.block_table, p.context_lens, p.ws,
                     p.counters);
  return hipGetLastError();
}

hipError_t launch_decode(int D, bool q_f32, int nrt, const DecodeArgs& a, const DecodePtrs& p,
                         hipStream_t stream) {
#define MQA_DEC(DD, QQ, NN) return launch_decode_t<DD, QQ, NN>(a, p, stream)
  if (D == 128) {
    if (q_f32) { if (nrt == 1) MQA_DEC(128, 2, 1); MQA_DEC(128, 2, 2); }
    if (nrt == 1) MQA_DEC(128, 1, 1);
    MQA_DEC(128, 1, 2);
  }
  if (q_f32) { if (nrt == 1) MQA_DEC(64, 2, 1); MQA_DEC(64, 2, 2); }
  if (nrt == 1) MQA_DEC(64, 1, 1);
  MQA_DEC(64, 1, 2);
#undef MQA_DEC
}

template <int D, int QS, int NRT>
static hipError_t launch_append_t(const AppendArgs& a, const AppendPtrs& p, hipStream_t stream) {
  hipLaunchKernelGGL((append_kernel<D, QS, NRT>), padded_grid(a.total_wgs), dim3(kAttnWaves * 64),
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
