// C-ABI entry points: descriptor normalisation, validation, workspace sizing and launches.
//
// Validation lives here, at the lowest callable boundary, and runs to completion before
// any launch.  TransformerEngine issue 1195 ("[PyTorch] fused CUDNN attention kernel not
// properly handling strides") is the failure this layer exists to prevent: the checks sat
// in a wrapper above the kernel modules, callers reached the modules directly, and packed
// q/k/v views were read as if contiguous.  Here every tensor is read through its own
// strides, the last stride must be 1, and outputs are proven disjoint or rejected.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <string>

#include <hip/hip_runtime_api.h>

#include "../../include/sdpa.h"
#include "launch.h"
#include "params.h"
#include "tiles.h"

using namespace sdpa;

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return SDPA_OK;
}

bool debug_enabled() {
  static int v = -1;
  if (v < 0) {
    const char* e = getenv("SDPA_DEBUG");
    v = (e && *e && strcmp(e, "0") != 0) ? 1 : 0;
  }
  return v == 1;
}

int esize_of(int32_t dtype) { return dtype == SDPA_DTYPE_F32 ? 4 : dtype == SDPA_DTYPE_FP8_E4M3 ? 1 : 2; }

// A tensor normalised to (batch, head, row, d) order: extents, element strides, base.
struct Norm {
  const char* name;
  const char* base;
  int esize;
  int64_t n[4];
  int64_t st[4];
  int64_t numel() const { return n[0] * n[1] * n[2] * n[3]; }
};

// Map the layout's logical stride order to (b, h, s, d).
void strides_bhsd(int32_t layout, const int64_t* in, int64_t* out) {
  switch (layout) {
    case SDPA_LAYOUT_BSHD: out[0] = in[0]; out[1] = in[2]; out[2] = in[1]; out[3] = in[3]; break;
    case SDPA_LAYOUT_SBHD: out[0] = in[1]; out[1] = in[2]; out[2] = in[0]; out[3] = in[3]; break;
    case SDPA_LAYOUT_BHSD: out[0] = in[0]; out[1] = in[1]; out[2] = in[2]; out[3] = in[3]; break;
    default: /* THD (t, h, d) */ out[0] = 0; out[1] = in[1]; out[2] = in[0]; out[3] = in[2]; break;
  }
}

Norm make_tensor(const char* name, const sdpa_tensor_t* t, int32_t layout, int esize,
                 int64_t b, int64_t h, int64_t s, int64_t d) {
  Norm r;
  r.name = name;
  r.base = static_cast<const char*>(t->data);
  r.esize = esize;
  r.n[0] = b; r.n[1] = h; r.n[2] = s; r.n[3] = d;
  strides_bhsd(layout, t->stride, r.st);
  return r;
}

Norm make_stat(const char* name, const sdpa_rowstat_t* t, bool thd, int64_t b, int64_t h,
               int64_t s) {
  Norm r;
  r.name = name;
  r.base = reinterpret_cast<const char*>(t->data);
  r.esize = 4;
  r.n[0] = b; r.n[1] = h; r.n[2] = s; r.n[3] = 1;
  if (thd) { r.st[0] = 0; r.st[1] = t->stride[0]; r.st[2] = t->stride[1]; }
  else { r.st[0] = t->stride[0]; r.st[1] = t->stride[1]; r.st[2] = t->stride[2]; }
  r.st[3] = 1;
  return r;
}

// Basic per-tensor checks: pointer, d-stride, sign, element alignment, offset range.
int check_tensor(const Norm& t, bool is_output, bool unit_last) {
  if (t.numel() == 0) return SDPA_OK;
  if (!t.base) return fail(SDPA_ERR_NULL, "%s: data pointer is NULL", t.name);
  if (unit_last && t.st[3] != 1)
    return fail(SDPA_ERR_STRIDE, "%s: the d (last) stride is %lld, it must be 1", t.name,
                (long long)t.st[3]);
  for (int i = 0; i < 4; ++i) {
    if (t.n[i] > 1 && t.st[i] < 0)
      return fail(SDPA_ERR_STRIDE, "%s: negative stride %lld", t.name, (long long)t.st[i]);
  }
  if (reinterpret_cast<uintptr_t>(t.base) % t.esize)
    return fail(SDPA_ERR_ALIGN, "%s: pointer not aligned to its %d-byte element", t.name, t.esize);
  // largest element offset must stay far from int64 overflow
  double span = 0;
  for (int i = 0; i < 4; ++i) span += double(t.n[i] - 1) * double(t.st[i] < 0 ? 0 : t.st[i]);
  if (span > 4.0e18 / t.esize) return fail(SDPA_ERR_SHAPE, "%s: addressed span too large", t.name);
  if (is_output) {
    // no two elements may share an address: with the active dims sorted by stride, each
    // stride must exceed the span of every smaller one.
    int idx[4], m = 0;
    for (int i = 0; i < 4; ++i)
      if (t.n[i] > 1) idx[m++] = i;
    std::sort(idx, idx + m, [&](int a, int b) { return t.st[a] < t.st[b]; });
    int64_t below = 0;
    for (int k = 0; k < m; ++k) {
      int64_t s = t.st[idx[k]];
      if (s <= below || s == 0)
        return fail(SDPA_ERR_STRIDE, "%s: output elements overlap (stride %lld over span %lld)",
                    t.name, (long long)s, (long long)below);
      below += (t.n[idx[k]] - 1) * s;
    }
  }
  return SDPA_OK;
}

void byte_span(const Norm& t, uintptr_t* lo, uintptr_t* hi) {
  int64_t last = 0;
  for (int i = 0; i < 4; ++i) last += (t.n[i] - 1) * t.st[i];
  *lo = reinterpret_cast<uintptr_t>(t.base);
  *hi = *lo + uintptr_t(last + 1) * t.esize;  // exclusive
}

int64_t floordiv(int64_t a, int64_t b) {
  int64_t q = a / b;
  if ((a % b != 0) && ((a < 0) != (b < 0))) --q;
  return q;
}

// True when A and B provably share no address.  Either their byte ranges are apart, or
// both are boxes of one non-overlapping parent with the same strides (e.g. disjoint head
// ranges of a packed [s, b, h_total, d] buffer, or disjoint row ranges of one tensor).
bool provably_disjoint(const Norm& a0, const Norm& b0) {
  if (a0.numel() == 0 || b0.numel() == 0) return true;
  // a dim of stride 0 (a broadcast input) addresses what extent 1 addresses
  Norm a = a0, b = b0;
  for (int i = 0; i < 4; ++i) {
    if (a.st[i] == 0) a.n[i] = 1;
    if (b.st[i] == 0) b.n[i] = 1;
  }
  uintptr_t alo, ahi, blo, bhi;
  byte_span(a, &alo, &ahi);
  byte_span(b, &blo, &bhi);
  if (ahi <= blo || bhi <= alo) return true;
  if (a.esize != b.esize) return false;
  int64_t diff = int64_t(blo) - int64_t(alo);
  if (diff % a.esize) return false;
  int64_t delta = diff / a.esize;
  int64_t st[4];
  int act[4], m = 0;
  for (int i = 0; i < 4; ++i) {
    bool aa = a.n[i] > 1, ba = b.n[i] > 1;
    if (!aa && !ba) continue;
    if (aa && ba && a.st[i] != b.st[i]) return false;
    st[i] = aa ? a.st[i] : b.st[i];
    if (st[i] <= 0) return false;
    act[m++] = i;
  }
  if (m == 0) return false;  // two single elements at the same address
  std::sort(act, act + m, [&](int x, int y) { return st[x] > st[y]; });
  // B's origin sits at coordinates c relative to A's: delta = sum_i c_i st_i.  Taking the
  // dims by decreasing stride, c_i is floor(rem / st_i) or one more (the smaller dims' part
  // of delta may be negative, e.g. B at a later head but an earlier row).  Any candidate
  // for which both boxes lie in one parent box whose addressing is injective (ascending
  // strides, each above the span of the smaller ones) and which keeps the boxes apart along
  // some dim is a proof: their elements sit at distinct coordinates of that box.
  for (int pick = 0; pick < (1 << m); ++pick) {
    int64_t c[4] = {0, 0, 0, 0};
    int64_t rem = delta;
    for (int k = 0; k < m; ++k) {
      c[act[k]] = floordiv(rem, st[act[k]]) + ((pick >> k) & 1);
      rem -= c[act[k]] * st[act[k]];
    }
    if (rem != 0) continue;
    bool injective = true;
    int64_t below = 0;
    for (int k = m - 1; k >= 0 && injective; --k) {
      int i = act[k];
      int64_t lo = std::min<int64_t>(0, c[i]);
      int64_t hi = std::max<int64_t>(a.n[i], c[i] + b.n[i]);
      if (st[i] <= below) injective = false;
      below += (hi - lo - 1) * st[i];
    }
    if (!injective) continue;
    for (int k = 0; k < m; ++k) {
      int i = act[k];
      if (c[i] >= a.n[i] || c[i] + b.n[i] <= 0) return true;  // boxes apart along dim i
    }
  }
  return false;
}

bool aligned16(const Norm& t) {
  if (t.numel() == 0) return true;
  if (reinterpret_cast<uintptr_t>(t.base) % 16) return false;
  for (int i = 0; i < 3; ++i)
    if (t.n[i] > 1 && (t.st[i] * t.esize) % 16) return false;
  return true;
}

View to_view(const Norm& t) {
  View v;
  v.ptr = const_cast<char*>(t.base);
  v.sb = t.st[0];
  v.sh = t.st[1];
  v.ss = t.st[2];
  return v;
}

StatView to_stat(const Norm& t) {
  StatView v;
  v.ptr = reinterpret_cast<float*>(const_cast<char*>(t.base));
  v.sb = t.st[0];
  v.sh = t.st[1];
  v.ss = t.st[2];
  return v;
}

int32_t clamp_rel(int64_t x) {
  return int32_t(std::max<int64_t>(-kUnbounded, std::min<int64_t>(kUnbounded, x)));
}

// Descriptor checks and the kernel-side Shape.
int check_desc(const sdpa_desc_t* d, Shape* s) {
  if (!d) return fail(SDPA_ERR_NULL, "desc is NULL");
  if (d->layout < 0 || d->layout > SDPA_LAYOUT_THD) return fail(SDPA_ERR_ARG, "layout %d out of range", d->layout);
  if (d->dtype < 0 || d->dtype > SDPA_DTYPE_FP8_E4M3) return fail(SDPA_ERR_ARG, "dtype %d out of range", d->dtype);
  if (d->diag_align != SDPA_ALIGN_TOP_LEFT && d->diag_align != SDPA_ALIGN_BOTTOM_RIGHT)
    return fail(SDPA_ERR_ARG, "diag_align %d out of range", d->diag_align);
  if (d->batch < 0 || d->seqlen_q < 0 || d->seqlen_k < 0)
    return fail(SDPA_ERR_SHAPE, "negative batch or sequence length");
  if (d->seqlen_q > kMaxSeqlen || d->seqlen_k > kMaxSeqlen)
    return fail(SDPA_ERR_SHAPE, "sequence length above %d", kMaxSeqlen);
  if (d->heads_q < 1 || d->heads_kv < 1 || d->heads_q > 65535)
    return fail(SDPA_ERR_SHAPE, "heads_q=%d heads_kv=%d", d->heads_q, d->heads_kv);
  if (d->heads_q % d->heads_kv)
    return fail(SDPA_ERR_SHAPE, "heads_q=%d is not a multiple of heads_kv=%d", d->heads_q, d->heads_kv);
  if (d->head_dim != 32 && d->head_dim != 64 && d->head_dim != 128)
    return fail(SDPA_ERR_UNSUPPORTED, "head_dim %d not built (32, 64, 128)", d->head_dim);
  if (!isfinite(d->softmax_scale)) return fail(SDPA_ERR_ARG, "softmax_scale is not finite");
  bool thd = d->layout == SDPA_LAYOUT_THD;
  if (thd) {
    if (d->batch > 0 && (!d->cu_seqlens_q || !d->cu_seqlens_k))
      return fail(SDPA_ERR_NULL, "THD needs cu_seqlens_q and cu_seqlens_k");
    if (d->total_q < 0 || d->total_k < 0 || d->total_q > INT32_MAX || d->total_k > INT32_MAX)
      return fail(SDPA_ERR_SHAPE, "total_q/total_k out of range");
  } else if (d->cu_seqlens_q_padded || d->cu_seqlens_k_padded) {
    return fail(SDPA_ERR_ARG, "cu_seqlens_*_padded are for the THD layout only");
  }
  {
    // every element count and byte size derived from the shape stays far from int64
    // overflow (workspace sizes and offsets are computed in int64)
    const double rq = (thd ? double(d->total_q) : double(d->batch) * d->seqlen_q) * d->heads_q;
    const double rk = (thd ? double(d->total_k) : double(d->batch) * d->seqlen_k) * d->heads_kv;
    if (std::max(rq, rk) * double(d->head_dim) * 8.0 > 4.0e18)
      return fail(SDPA_ERR_SHAPE, "problem too large: %.3g query rows, %.3g key rows", rq, rk);
  }
  const sdpa_block_mask_t* m = d->block_mask;
  if (m) {
    if (thd) return fail(SDPA_ERR_UNSUPPORTED, "block_mask is for the BSHD, SBHD and BHSD layouts");
    if (!m->bits || !m->kv_count || !m->kv_list || !m->q_count || !m->q_list)
      return fail(SDPA_ERR_NULL, "block_mask has a NULL array");
    if ((m->batch != 1 && m->batch != d->batch) || (m->heads != 1 && m->heads != d->heads_q))
      return fail(SDPA_ERR_SHAPE, "block_mask batch=%d heads=%d (1 or batch=%d / heads_q=%d)",
                  m->batch, m->heads, d->batch, d->heads_q);
    if ((d->seqlen_k + kMaskBlock - 1) / kMaskBlock > kMaskMaxList ||
        (d->seqlen_q + kMaskBlock - 1) / kMaskBlock > kMaskMaxList)
      return fail(SDPA_ERR_UNSUPPORTED, "block_mask with seqlen_q %d / seqlen_k %d above %d",
                  d->seqlen_q, d->seqlen_k, kMaskMaxList * kMaskBlock);
  }
  memset(s, 0, sizeof(*s));
  if (m) {
    s->bm.bits = m->bits;
    s->bm.kv_count = m->kv_count;
    s->bm.kv_list = m->kv_list;
    s->bm.q_count = m->q_count;
    s->bm.q_list = m->q_list;
    s->bm.nb = m->batch;
    s->bm.nh = m->heads;
    s->bm.nqb = (d->seqlen_q + kMaskBlock - 1) / kMaskBlock;
    s->bm.nkb = (d->seqlen_k + kMaskBlock - 1) / kMaskBlock;
    s->bm.words = (d->seqlen_k + 63) / 64;
  }
  s->batch = d->batch;
  s->sq = d->seqlen_q;
  s->sk = d->seqlen_k;
  s->hq = d->heads_q;
  s->hk = d->heads_kv;
  s->group = d->heads_q / d->heads_kv;
  s->d = d->head_dim;
  s->thd = thd;
  s->cu_q = d->cu_seqlens_q;
  s->cu_k = d->cu_seqlens_k;
  s->pad_q = thd ? d->cu_seqlens_q_padded : nullptr;
  s->pad_k = thd ? d->cu_seqlens_k_padded : nullptr;
  s->total_q = thd ? d->total_q : 0;
  s->total_k = thd ? d->total_k : 0;
  s->lo_rel = d->window_left == -1 ? -kUnbounded : clamp_rel(-int64_t(d->window_left));
  s->hi_rel = d->window_right == -1 ? kUnbounded : clamp_rel(int64_t(d->window_right));
  s->bottom_right = d->diag_align == SDPA_ALIGN_BOTTOM_RIGHT;
  {
    const int64_t off = s->bottom_right ? int64_t(s->sk) - s->sq : 0;
    s->uniform = !thd && !s->bm.bits && int64_t(s->sq) - 1 + off + s->lo_rel <= 0 &&
                 int64_t(s->hi_rel) + off >= int64_t(s->sk) - 1;
  }
  s->scale = d->softmax_scale;
  s->scale_log2 = float(double(d->softmax_scale) * 1.4426950408889634);
  {
    // The tile kernels launch at most 4 work-items per query and per key row, rows padded to
    // 128-row tiles per (sequence, head), and a dispatch counts work-items in 32 bits: refuse
    // here what no grid could cover, before any launch (double: the products of extreme
    // descriptor values overflow 64 bits)
    auto padded = [&](double rows, double heads) {
      return thd ? heads * (rows + double(d->batch) * 128)
                 : heads * double(d->batch) * ceil(rows / 128) * 128;
    };
    const double pq = padded(thd ? double(d->total_q) : double(d->seqlen_q), d->heads_q);
    const double pk = padded(thd ? double(d->total_k) : double(d->seqlen_k), d->heads_kv);
    if (4 * (pq + pk) > double(kMaxGridItems))
      return fail(SDPA_ERR_UNSUPPORTED,
                  "problem too large: %.0f padded query and key rows over all heads, at most %lld",
                  pq + pk, (long long)(kMaxGridItems / 4));
  }
  return SDPA_OK;
}

struct Attn {
  Shape s;
  int64_t rows_q, rows_k, nb;  // per-tensor row extents and batch extent
  int32_t layout, dtype;
};

int attn_setup(const sdpa_desc_t* d, Attn* a) {
  int rc = check_desc(d, &a->s);
  if (rc) return rc;
  bool thd = a->s.thd;
  a->layout = d->layout;
  a->dtype = d->dtype;
  a->nb = thd ? 1 : d->batch;
  a->rows_q = thd ? d->total_q : d->seqlen_q;
  a->rows_k = thd ? d->total_k : d->seqlen_k;
  return SDPA_OK;
}

Norm qlike(const Attn& a, const char* name, const sdpa_tensor_t* t) {
  return make_tensor(name, t, a.layout, esize_of(a.dtype), a.nb, a.s.hq, a.rows_q, a.s.d);
}
Norm klike(const Attn& a, const char* name, const sdpa_tensor_t* t) {
  return make_tensor(name, t, a.layout, esize_of(a.dtype), a.nb, a.s.hk, a.rows_k, a.s.d);
}
Norm statlike(const Attn& a, const char* name, const sdpa_rowstat_t* t) {
  return make_stat(name, t, a.s.thd, a.nb, a.s.hq, a.rows_q);
}

int check_outputs(const Norm* outs, int nout, const Norm* ins, int nin) {
  for (int i = 0; i < nout; ++i) {
    for (int j = i + 1; j < nout; ++j)
      if (!provably_disjoint(outs[i], outs[j]))
        return fail(SDPA_ERR_ALIAS, "outputs %s and %s may overlap", outs[i].name, outs[j].name);
    for (int j = 0; j < nin; ++j)
      if (!provably_disjoint(outs[i], ins[j]))
        return fail(SDPA_ERR_ALIAS, "output %s may overlap input %s", outs[i].name, ins[j].name);
  }
  return SDPA_OK;
}

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

int64_t thd_items(int64_t total, int32_t batch, int tile) {
  return (total + tile - 1) / tile + batch;
}

int fwd_rows_per_tile(int32_t dtype) { return dtype == SDPA_DTYPE_F32 ? kFwdBM : kFwdBM16; }

size_t fwd_ws_bytes(const Shape& s, int32_t dtype) {
  if (!s.thd) return 0;
  const int bm = fwd_rows_per_tile(dtype);
  return size_t(round_up(thd_items(s.total_q, s.batch, bm) * int64_t(sizeof(WorkItem)), 256) + 256);
}

struct BwdWs {
  int64_t delta_off, lse2_off, wq_off, cq_off, wk_off, ck_off, total;
  int64_t split_blocks, cnt_off, part_off;  // split dK/dV (split_blocks = 0: none)
  int64_t ksplit_cap, kcnt_off, kpart_off;  // split THD dK/dV items (ksplit_cap = 0: none)
};

int bwd_q_rows(int32_t dtype) { return dtype == SDPA_DTYPE_F32 ? kBwdQ32 : kBwdQ16; }
int bwd_k_rows(int32_t dtype) { return dtype == SDPA_DTYPE_F32 ? kBwdK32 : kBwdK16; }


// Split dK/dV blocks: GQA groups, 16-bit inputs, head_dim 64 or 128, no block mask, and a
// small grid (at most kBwdSplitPerCU dK/dV plus dQ blocks per CU of the current device),
// where the longest dK/dV chain (G times the longest dQ chain) sets the time.  On larger
// grids the extra blocks and the partial sums cost more than the shorter chain saves.
bool bwd_split_ok(const Shape& s, int32_t dtype) {
  if (s.group < 2 || dtype == SDPA_DTYPE_F32 || dtype == SDPA_DTYPE_FP8_E4M3 ||
      (s.d != 64 && s.d != 128) || s.bm.bits)
    return false;
  const int64_t tk = kBwdK16, tq = kBwdQ16;
  const int64_t nk = s.thd ? ((s.total_k + tk - 1) / tk + s.batch) * s.hk
                           : ((s.sk + tk - 1) / tk) * int64_t(s.batch) * s.hk;
  const int64_t nq = s.thd ? ((s.total_q + tq - 1) / tq + s.batch) * s.hq
                           : ((s.sq + tq - 1) / tq) * int64_t(s.batch) * s.hq;
  return nk + nq <= int64_t(kBwdSplitPerCU) * device_cus() && nk * 2 < (int64_t(1) << 30);
}

// THD, 16-bit, head_dim 64 or 128, no block mask, on a grid large enough for the separate
// dK/dV launch (more than kBwdWideMinPerCU fused blocks per CU): room for the partial sums of
// split items, 2 halves x 128 keys x D x {dK, dV} in fp32 per item and kv head, up to 32 MiB
// (at most 64 items).  The launcher decides on the strides whether the launch is used.
int64_t bwd_ksplit_cap(const Shape& s, int32_t dtype) {
  if (!s.thd || dtype == SDPA_DTYPE_F32 || dtype == SDPA_DTYPE_FP8_E4M3 || (s.d != 64 && s.d != 128) ||
      s.bm.bits || s.hk < 1)
    return 0;
  const int64_t tk = kBwdK16, tq = kBwdQ16;
  const int64_t nk = ((s.total_k + tk - 1) / tk + s.batch) * s.hk;
  const int64_t nq = ((s.total_q + tq - 1) / tq + s.batch) * s.hq;
  if (nq + nk <= int64_t(kBwdWideMinPerCU) * device_cus()) return 0;
  const int64_t per = int64_t(s.hk) * 2 * kBwdK16Wide * s.d * 2 * 4;
  return std::max<int64_t>(1, std::min<int64_t>(64, (int64_t(32) << 20) / per));
}

// split_area = false: the layout without room for split THD dK/dV items (the backward then
// splits none); a workspace of at least that size still runs.
BwdWs bwd_ws_layout(const Shape& s, int32_t dtype, bool split_area = true) {
  BwdWs w{};
  int64_t rows = s.thd ? int64_t(s.hq) * s.total_q : int64_t(s.batch) * s.hq * s.sq;
  w.delta_off = 0;
  w.lse2_off = round_up(rows * 4, 256);
  int64_t off = round_up(w.lse2_off + rows * 4, 256);
  w.ksplit_cap = split_area ? bwd_ksplit_cap(s, dtype) : 0;
  if (s.thd) {
    w.wq_off = off;
    off = round_up(off + thd_items(s.total_q, s.batch, bwd_q_rows(dtype)) * int64_t(sizeof(WorkItem)), 256);
    w.cq_off = off;
    off += 256;
    w.wk_off = off;  // (a split item takes two entries)
    off = round_up(off + (thd_items(s.total_k, s.batch, bwd_k_rows(dtype)) + w.ksplit_cap) * int64_t(sizeof(WorkItem)), 256);
    w.ck_off = off;
    off += 256;
  }
  // GQA on the fused 16-bit backward: every dK/dV block runs as two halves whose fp32
  // partial sums (2 halves x 64 keys x D x {dK, dV}) meet in the workspace
  if (bwd_split_ok(s, dtype)) {
    const int64_t tk = kBwdK16;
    w.split_blocks = s.thd ? ((s.total_k + tk - 1) / tk + s.batch) * s.hk
                           : ((s.sk + tk - 1) / tk) * int64_t(s.batch) * s.hk;
    w.cnt_off = off;
    off = round_up(off + w.split_blocks * 4, 256);
    w.part_off = off;
    off = round_up(off + w.split_blocks * 2 * 64 * int64_t(s.d) * 2 * 4, 256);
  }
  if (w.ksplit_cap > 0) {
    w.kcnt_off = off;
    off += 256;
    w.kpart_off = off;
    off = round_up(off + w.ksplit_cap * s.hk * 2 * kBwdK16Wide * int64_t(s.d) * 2 * 4, 256);
  }
  w.total = off;
  return w;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(SDPA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Validation shared by sdpa_fwd and sdpa_fwd_validate.
int fwd_check(const sdpa_desc_t* desc, const sdpa_tensor_t* q, const sdpa_tensor_t* k,
              const sdpa_tensor_t* v, const sdpa_tensor_t* o, const sdpa_rowstat_t* lse,
              size_t ws_bytes, Attn* a, FwdParams* p, bool fp8 = false) {
  int rc = attn_setup(desc, a);
  if (rc) return rc;
  if ((a->dtype == SDPA_DTYPE_FP8_E4M3) != fp8)
    return fail(SDPA_ERR_UNSUPPORTED, fp8 ? "sdpa_fwd_fp8 needs dtype SDPA_DTYPE_FP8_E4M3"
                                          : "FP8 inputs take sdpa_fwd_fp8 (forward only)");
  if (fp8 && a->s.bm.bits) return fail(SDPA_ERR_UNSUPPORTED, "sdpa_fwd_fp8 takes no block_mask");
  if (!q || !k || !v || !o || !lse) return fail(SDPA_ERR_NULL, "a tensor handle is NULL");
  Norm nq = qlike(*a, "q", q), nk = klike(*a, "k", k), nv = klike(*a, "v", v);
  // FP8: o is bf16
  Norm no = fp8 ? make_tensor("o", o, a->layout, 2, a->nb, a->s.hq, a->rows_q, a->s.d) : qlike(*a, "o", o);
  Norm nl = statlike(*a, "lse", lse);
  bool has_lse = lse->data != nullptr;
  if ((rc = check_tensor(nq, false, true)) || (rc = check_tensor(nk, false, true)) ||
      (rc = check_tensor(nv, false, true)) || (rc = check_tensor(no, true, true)))
    return rc;
  if (has_lse && (rc = check_tensor(nl, true, false))) return rc;
  Norm outs[2] = {no, nl};
  Norm ins[3] = {nq, nk, nv};
  if ((rc = check_outputs(outs, has_lse ? 2 : 1, ins, 3))) return rc;
  size_t need = fwd_ws_bytes(a->s, a->dtype);
  if (need && ws_bytes < need)
    return fail(SDPA_ERR_WORKSPACE, "workspace %zu bytes, %zu needed", ws_bytes, need);
  const int bm = fwd_rows_per_tile(a->dtype);
  int64_t blocks = a->s.thd ? thd_items(a->s.total_q, a->s.batch, bm) * a->s.hq
                            : int64_t((a->s.sq + bm - 1) / bm) * a->s.batch * a->s.hq;
  if (blocks > INT32_MAX) return fail(SDPA_ERR_SHAPE, "problem too large for one launch");
  memset(p, 0, sizeof(*p));
  p->s = a->s;
  p->q = to_view(nq);
  p->k = to_view(nk);
  p->v = to_view(nv);
  p->o = to_view(no);
  p->lse = to_stat(nl);
  if (!has_lse) p->lse.ptr = nullptr;
  p->aligned = (aligned16(nq) ? kAlQ : 0) | (aligned16(nk) ? kAlK : 0) |
               (aligned16(nv) ? kAlV : 0) | (aligned16(no) ? kAlO : 0);
  if (fp8 && !fwd8_ok(*p))
    return fail(SDPA_ERR_UNSUPPORTED,
                "FP8 forward needs head_dim 64 or 128 and 16-byte aligned q/k/v/o rows with k/v "
                "row strides >= head_dim");
  if (p->s.bm.bits && !fwd_block_mask_ok(*p, DType(a->dtype)))
    return fail(SDPA_ERR_UNSUPPORTED,
                "block_mask needs 16-byte aligned q/k/v/o rows with k/v row strides >= head_dim "
                "for 16-bit inputs");
  return SDPA_OK;
}

int bwd_check(const sdpa_desc_t* desc, const sdpa_tensor_t* q, const sdpa_tensor_t* k,
              const sdpa_tensor_t* v, const sdpa_tensor_t* o, const sdpa_rowstat_t* lse,
              const sdpa_tensor_t* dout, const sdpa_rowstat_t* dlse, const sdpa_tensor_t* dq,
              const sdpa_tensor_t* dk, const sdpa_tensor_t* dv, size_t ws_bytes, Attn* a,
              BwdParams* p) {
  int rc = attn_setup(desc, a);
  if (rc) return rc;
  if (a->dtype == SDPA_DTYPE_FP8_E4M3) return fail(SDPA_ERR_UNSUPPORTED, "FP8 inputs: forward only");
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv)
    return fail(SDPA_ERR_NULL, "a tensor handle is NULL");
  Norm nq = qlike(*a, "q", q), nk = klike(*a, "k", k), nv = klike(*a, "v", v);
  Norm no = qlike(*a, "o", o), ndo = qlike(*a, "dout", dout);
  Norm nl = statlike(*a, "lse", lse);
  bool has_dlse = dlse && dlse->data;
  Norm ndl = has_dlse ? statlike(*a, "dlse", dlse) : nl;
  Norm ndq = qlike(*a, "dq", dq), ndk = klike(*a, "dk", dk), ndv = klike(*a, "dv", dv);
  if ((rc = check_tensor(nq, false, true)) || (rc = check_tensor(nk, false, true)) ||
      (rc = check_tensor(nv, false, true)) || (rc = check_tensor(no, false, true)) ||
      (rc = check_tensor(ndo, false, true)) || (rc = check_tensor(nl, false, false)) ||
      (rc = check_tensor(ndq, true, true)) || (rc = check_tensor(ndk, true, true)) ||
      (rc = check_tensor(ndv, true, true)))
    return rc;
  if (has_dlse && (rc = check_tensor(ndl, false, false))) return rc;
  Norm outs[3] = {ndq, ndk, ndv};
  Norm ins[7] = {nq, nk, nv, no, ndo, nl, ndl};
  if ((rc = check_outputs(outs, 3, ins, has_dlse ? 7 : 6))) return rc;
  BwdWs w = bwd_ws_layout(a->s, a->dtype);
  if (ws_bytes < size_t(w.total)) w = bwd_ws_layout(a->s, a->dtype, false);  // no split room
  if (ws_bytes < size_t(w.total))
    return fail(SDPA_ERR_WORKSPACE, "workspace %zu bytes, %lld needed", ws_bytes, (long long)w.total);
  memset(p, 0, sizeof(*p));
  p->s = a->s;
  p->q = to_view(nq); p->k = to_view(nk); p->v = to_view(nv); p->o = to_view(no);
  p->dout = to_view(ndo); p->dq = to_view(ndq); p->dk = to_view(ndk); p->dv = to_view(ndv);
  p->lse = to_stat(nl);
  p->dlse = to_stat(ndl);
  if (!has_dlse) p->dlse.ptr = nullptr;
  p->aligned = (aligned16(nq) ? kAlQ : 0) | (aligned16(nk) ? kAlK : 0) |
               (aligned16(nv) ? kAlV : 0) | (aligned16(no) ? kAlO : 0) |
               (aligned16(ndo) ? kAlDO : 0) | (aligned16(ndq) ? kAlDQ : 0) |
               (aligned16(ndk) ? kAlDK : 0) | (aligned16(ndv) ? kAlDV : 0);
  if (p->s.bm.bits && !bwd_block_mask_ok(*p, DType(a->dtype)))
    return fail(SDPA_ERR_UNSUPPORTED,
                "block_mask backward needs head_dim >= 64 and 16-byte aligned rows with row "
                "strides >= head_dim for 16-bit inputs");
  return SDPA_OK;
}

void debug_log(const char* call, const Attn& a, const void* extra) {
  if (!debug_enabled()) return;
  const Shape& s = a.s;
  fprintf(stderr,
          "[sdpa] %s layout=%d dtype=%d B=%d Sq=%d Sk=%d Hq=%d Hk=%d D=%d thd=%d "
          "rel=[%d,%d] br=%d scale=%g aligned=0x%x\n",
          call, a.layout, a.dtype, s.batch, s.sq, s.sk, s.hq, s.hk, s.d, s.thd, s.lo_rel, s.hi_rel,
          s.bottom_right, double(s.scale), extra ? *static_cast<const int*>(extra) : -1);
}

// ---------------------------------------------------------------------------------------
// merge
// ---------------------------------------------------------------------------------------

struct Merge {
  int64_t nb, h, rows, d;
  int32_t layout, dtype;
  bool thd;
  const int32_t* cu = nullptr;   // THD sequence map (optional)
  const int32_t* pad = nullptr;
  int32_t nseq = 0;
};

int merge_setup(const sdpa_merge_desc_t* d, Merge* m) {
  if (!d) return fail(SDPA_ERR_NULL, "merge desc is NULL");
  if (d->layout < 0 || d->layout > SDPA_LAYOUT_THD) return fail(SDPA_ERR_ARG, "layout out of range");
  if (d->dtype < 0 || d->dtype > SDPA_DTYPE_FP8_E4M3) return fail(SDPA_ERR_ARG, "dtype out of range");
  if (d->dtype == SDPA_DTYPE_FP8_E4M3) return fail(SDPA_ERR_UNSUPPORTED, "the merge takes fp16, bf16 or fp32");
  if (d->head_dim != 32 && d->head_dim != 64 && d->head_dim != 128)
    return fail(SDPA_ERR_UNSUPPORTED, "head_dim %d not built (32, 64, 128)", d->head_dim);
  m->thd = d->layout == SDPA_LAYOUT_THD;
  if (d->heads < 1 || d->heads > 65535) return fail(SDPA_ERR_SHAPE, "heads=%d", d->heads);
  if (m->thd) {
    if (d->total < 0 || d->total > INT32_MAX) return fail(SDPA_ERR_SHAPE, "total out of range");
    if (d->cu_seqlens && d->batch < 0) return fail(SDPA_ERR_SHAPE, "batch out of range");
    if (!d->cu_seqlens && d->cu_seqlens_padded)
      return fail(SDPA_ERR_NULL, "cu_seqlens_padded without cu_seqlens");
  } else if (d->batch < 0 || d->seqlen < 0 || d->seqlen > kMaxSeqlen) {
    return fail(SDPA_ERR_SHAPE, "batch/seqlen out of range");
  } else if (d->cu_seqlens || d->cu_seqlens_padded) {
    return fail(SDPA_ERR_ARG, "cu_seqlens in a merge are for the THD layout only");
  }
  m->cu = m->thd ? d->cu_seqlens : nullptr;
  m->pad = m->thd ? d->cu_seqlens_padded : nullptr;
  m->nseq = d->batch;
  m->layout = d->layout;
  m->dtype = d->dtype;
  m->nb = m->thd ? 1 : d->batch;
  m->h = d->heads;
  m->rows = m->thd ? d->total : d->seqlen;
  m->d = d->head_dim;
  return SDPA_OK;
}

Norm mx(const Merge& m, const char* name, const sdpa_tensor_t* t) {
  return make_tensor(name, t, m.layout, esize_of(m.dtype), m.nb, m.h, m.rows, m.d);
}
Norm ml(const Merge& m, const char* name, const sdpa_rowstat_t* t) {
  return make_stat(name, t, m.thd, m.nb, m.h, m.rows);
}

void merge_params(const Merge& m, MergeParams* p) {
  memset(p, 0, sizeof(*p));
  p->rows = m.nb * m.h * m.rows;
  p->batch = int32_t(m.nb);
  p->seqlen = int32_t(m.rows);
  p->heads = int32_t(m.h);
  p->d = int32_t(m.d);
  p->thd = m.thd;
  p->cu = m.cu;
  p->pad = m.pad;
  p->nseq = m.cu ? m.nseq : 0;
}

int merge_fwd_check(const sdpa_merge_desc_t* desc, const sdpa_tensor_t* xa,
                    const sdpa_rowstat_t* la, const sdpa_tensor_t* xb, const sdpa_rowstat_t* lb,
                    const sdpa_tensor_t* x, const sdpa_rowstat_t* l, Merge* m, MergeParams* p) {
  int rc = merge_setup(desc, m);
  if (rc) return rc;
  if (!xa || !la || !xb || !lb || !x || !l) return fail(SDPA_ERR_NULL, "a tensor handle is NULL");
  Norm nxa = mx(*m, "x_a", xa), nxb = mx(*m, "x_b", xb), nx = mx(*m, "x", x);
  Norm nla = ml(*m, "lse_a", la), nlb = ml(*m, "lse_b", lb), nl = ml(*m, "lse", l);
  bool has_l = l->data != nullptr;
  if ((rc = check_tensor(nxa, false, true)) || (rc = check_tensor(nxb, false, true)) ||
      (rc = check_tensor(nx, true, true)) || (rc = check_tensor(nla, false, false)) ||
      (rc = check_tensor(nlb, false, false)))
    return rc;
  if (has_l && (rc = check_tensor(nl, true, false))) return rc;
  Norm outs[2] = {nx, nl};
  Norm ins[4] = {nxa, nxb, nla, nlb};
  if ((rc = check_outputs(outs, has_l ? 2 : 1, ins, 4))) return rc;
  merge_params(*m, p);
  p->xa = to_view(nxa); p->xb = to_view(nxb); p->x = to_view(nx);
  p->la = to_stat(nla); p->lb = to_stat(nlb); p->l = to_stat(nl);
  if (!has_l) p->l.ptr = nullptr;
  p->aligned = aligned16(nxa) && aligned16(nxb) && aligned16(nx);
  return SDPA_OK;
}

int merge_bwd_check(const sdpa_merge_desc_t* desc, const sdpa_tensor_t* xa,
                    const sdpa_rowstat_t* la, const sdpa_tensor_t* xb, const sdpa_rowstat_t* lb,
                    const sdpa_tensor_t* g, const sdpa_rowstat_t* gl, const sdpa_tensor_t* dxa,
                    const sdpa_rowstat_t* dla, const sdpa_tensor_t* dxb,
                    const sdpa_rowstat_t* dlb, Merge* m, MergeParams* p) {
  int rc = merge_setup(desc, m);
  if (rc) return rc;
  if (!xa || !la || !xb || !lb || !g || !dxa || !dla || !dxb || !dlb)
    return fail(SDPA_ERR_NULL, "a tensor handle is NULL");
  Norm nxa = mx(*m, "x_a", xa), nxb = mx(*m, "x_b", xb), ng = mx(*m, "g", g);
  Norm ndxa = mx(*m, "dx_a", dxa), ndxb = mx(*m, "dx_b", dxb);
  Norm nla = ml(*m, "lse_a", la), nlb = ml(*m, "lse_b", lb);
  Norm ndla = ml(*m, "dlse_a", dla), ndlb = ml(*m, "dlse_b", dlb);
  bool has_gl = gl && gl->data;
  Norm ngl = has_gl ? ml(*m, "g_lse", gl) : nla;
  if ((rc = check_tensor(nxa, false, true)) || (rc = check_tensor(nxb, false, true)) ||
      (rc = check_tensor(ng, false, true)) || (rc = check_tensor(ndxa, true, true)) ||
      (rc = check_tensor(ndxb, true, true)) || (rc = check_tensor(nla, false, false)) ||
      (rc = check_tensor(nlb, false, false)) || (rc = check_tensor(ndla, true, false)) ||
      (rc = check_tensor(ndlb, true, false)))
    return rc;
  if (has_gl && (rc = check_tensor(ngl, false, false))) return rc;
  Norm outs[4] = {ndxa, ndxb, ndla, ndlb};
  Norm ins[6] = {nxa, nxb, ng, nla, nlb, ngl};
  if ((rc = check_outputs(outs, 4, ins, has_gl ? 6 : 5))) return rc;
  merge_params(*m, p);
  p->xa = to_view(nxa); p->xb = to_view(nxb); p->g = to_view(ng);
  p->dxa = to_view(ndxa); p->dxb = to_view(ndxb);
  p->la = to_stat(nla); p->lb = to_stat(nlb); p->glse = to_stat(ngl);
  p->dla = to_stat(ndla); p->dlb = to_stat(ndlb);
  if (!has_gl) p->glse.ptr = nullptr;
  p->aligned = aligned16(nxa) && aligned16(nxb) && aligned16(ng) && aligned16(ndxa) &&
               aligned16(ndxb);
  return SDPA_OK;
}

SchedParams sched_params(const Shape& s, bool q_items, WorkItem* items, int32_t* count) {
  SchedParams sp;
  memset(&sp, 0, sizeof(sp));
  sp.cu_own = q_items ? s.cu_q : s.cu_k;
  sp.cu_other = q_items ? s.cu_k : s.cu_q;
  sp.total_own = q_items ? s.total_q : s.total_k;
  sp.total_other = q_items ? s.total_k : s.total_q;
  sp.batch = s.batch;
  sp.max_own = q_items ? s.sq : s.sk;
  sp.max_other = q_items ? s.sk : s.sq;
  sp.lo_rel = s.lo_rel;
  sp.hi_rel = s.hi_rel;
  sp.bottom_right = s.bottom_right;
  sp.own_is_query = q_items;
  sp.items = items;
  sp.count = count;
  return sp;
}

}  // namespace

namespace sdpa {
// Compute units of the current device (0 if unknown), cached per device.
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      return 0;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Record an error message for sdpa_last_error() from another translation unit.
int set_error(int code, const char* msg) { return fail(code, "%s", msg); }

// The smallest backward workspace for desc: without room for split THD dK/dV items.
int bwd_workspace_min(const sdpa_desc_t* desc, size_t* bytes) {
  Shape s;
  int rc = check_desc(desc, &s);
  if (rc) return rc;
  *bytes = size_t(bwd_ws_layout(s, desc->dtype, false).total);
  return ok();
}
int clear_error() { return ok(); }
}  // namespace sdpa

extern "C" {

int sdpa_version(void) { return SDPA_VERSION; }

const char* sdpa_last_error(void) { return g_last_error.c_str(); }

int sdpa_fwd_workspace_size(const sdpa_desc_t* desc, size_t* bytes) {
  Shape s;
  int rc = check_desc(desc, &s);
  if (rc) return rc;
  if (!bytes) return fail(SDPA_ERR_NULL, "bytes is NULL");
  *bytes = fwd_ws_bytes(s, desc->dtype);
  return ok();
}

int sdpa_fwd_validate(const sdpa_desc_t* desc, const sdpa_tensor_t* q, const sdpa_tensor_t* k,
                      const sdpa_tensor_t* v, const sdpa_tensor_t* o, const sdpa_rowstat_t* lse,
                      size_t workspace_bytes) {
  Attn a;
  FwdParams p;
  int rc = fwd_check(desc, q, k, v, o, lse, workspace_bytes, &a, &p);
  return rc ? rc : ok();
}

int sdpa_fwd(const sdpa_desc_t* desc, const sdpa_tensor_t* q, const sdpa_tensor_t* k,
             const sdpa_tensor_t* v, const sdpa_tensor_t* o, const sdpa_rowstat_t* lse,
             void* workspace, size_t workspace_bytes, void* stream) {
  Attn a;
  FwdParams p;
  int rc = fwd_check(desc, q, k, v, o, lse, workspace_bytes, &a, &p);
  if (rc) return rc;
  size_t need = fwd_ws_bytes(a.s, a.dtype);
  if (need && !workspace) return fail(SDPA_ERR_WORKSPACE, "THD forward needs a workspace");
  debug_log("fwd", a, &p.aligned);
  if (a.s.batch == 0 || a.rows_q == 0) return ok();
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (a.s.thd) {
    char* ws = static_cast<char*>(workspace);
    const int bm = fwd_rows_per_tile(a.dtype);
    int64_t nitems = thd_items(a.s.total_q, a.s.batch, bm);
    WorkItem* items = reinterpret_cast<WorkItem*>(ws);
    int32_t* count = reinterpret_cast<int32_t*>(ws + need - 256);
    SchedParams sp = sched_params(a.s, true, items, count);
    sp.tile_own = bm;
    sp.tile_other = a.dtype == SDPA_DTYPE_F32 ? kFwdBN32 : kFwdBN16;
    sp.max_items = int32_t(nitems);
    if ((e = launch_schedule(sp, st)) != hipSuccess) return hip_fail(e, "THD schedule launch");
    p.work = items;
    p.work_count = count;
  }
  if ((e = launch_fwd(p, DType(a.dtype), st)) != hipSuccess) return hip_fail(e, "forward launch");
  return ok();
}

int sdpa_fwd_fp8_validate(const sdpa_desc_t* desc, const sdpa_tensor_t* q, const sdpa_tensor_t* k,
                          const sdpa_tensor_t* v, const sdpa_tensor_t* o, const sdpa_rowstat_t* lse,
                          size_t workspace_bytes) {
  Attn a;
  FwdParams p;
  int rc = fwd_check(desc, q, k, v, o, lse, workspace_bytes, &a, &p, true);
  return rc ? rc : ok();
}

int sdpa_fwd_fp8(const sdpa_desc_t* desc, const sdpa_tensor_t* q, const sdpa_tensor_t* k,
                 const sdpa_tensor_t* v, const float* descale_q, const float* descale_k,
                 const float* descale_v, const sdpa_tensor_t* o, const sdpa_rowstat_t* lse,
                 void* workspace, size_t workspace_bytes, void* stream) {
  Attn a;
  FwdParams p;
  int rc = fwd_check(desc, q, k, v, o, lse, workspace_bytes, &a, &p, true);
  if (rc) return rc;
  size_t need = fwd_ws_bytes(a.s, a.dtype);
  if (need && !workspace) return fail(SDPA_ERR_WORKSPACE, "THD forward needs a workspace");
  p.descale_q = descale_q;
  p.descale_k = descale_k;
  p.descale_v = descale_v;
  debug_log("fwd_fp8", a, &p.aligned);
  if (a.s.batch == 0 || a.rows_q == 0) return ok();
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (a.s.thd) {
    char* ws = static_cast<char*>(workspace);
    const int bm = fwd_rows_per_tile(a.dtype);
    int64_t nitems = thd_items(a.s.total_q, a.s.batch, bm);
    WorkItem* items = reinterpret_cast<WorkItem*>(ws);
    int32_t* count = reinterpret_cast<int32_t*>(ws + need - 256);
    SchedParams sp = sched_params(a.s, true, items, count);
    sp.tile_own = bm;
    sp.tile_other = kFwdBN16;
    sp.max_items = int32_t(nitems);
    if ((e = launch_schedule(sp, st)) != hipSuccess) return hip_fail(e, "THD schedule launch");
    p.work = items;
    p.work_count = count;
  }
  if ((e = launch_fwd8(p, st)) != hipSuccess) return hip_fail(e, "FP8 forward launch");
  return ok();
}

int sdpa_bwd_workspace_size(const sdpa_desc_t* desc, size_t* bytes) {
  Shape s;
  int rc = check_desc(desc, &s);
  if (rc) return rc;
  if (!bytes) return fail(SDPA_ERR_NULL, "bytes is NULL");
  *bytes = size_t(bwd_ws_layout(s, desc->dtype).total);
  return ok();
}

int sdpa_bwd_validate(const sdpa_desc_t* desc, const sdpa_tensor_t* q, const sdpa_tensor_t* k,
                      const sdpa_tensor_t* v, const sdpa_tensor_t* o, const sdpa_rowstat_t* lse,
                      const sdpa_tensor_t* dout, const sdpa_rowstat_t* dlse,
                      const sdpa_tensor_t* dq, const sdpa_tensor_t* dk, const sdpa_tensor_t* dv,
                      size_t workspace_bytes) {
  Attn a;
  BwdParams p;
  int rc = bwd_check(desc, q, k, v, o, lse, dout, dlse, dq, dk, dv, workspace_bytes, &a, &p);
  return rc ? rc : ok();
}

int sdpa_bwd(const sdpa_desc_t* desc, const sdpa_tensor_t* q, const sdpa_tensor_t* k,
             const sdpa_tensor_t* v, const sdpa_tensor_t* o, const sdpa_rowstat_t* lse,
             const sdpa_tensor_t* dout, const sdpa_rowstat_t* dlse, const sdpa_tensor_t* dq,
             const sdpa_tensor_t* dk, const sdpa_tensor_t* dv, int accumulate, void* workspace,
             size_t workspace_bytes, void* stream) {
  Attn a;
  BwdParams p;
  int rc = bwd_check(desc, q, k, v, o, lse, dout, dlse, dq, dk, dv, workspace_bytes, &a, &p);
  if (rc) return rc;
  if (accumulate != 0 && accumulate != 1) return fail(SDPA_ERR_ARG, "accumulate must be 0 or 1");
  BwdWs w = bwd_ws_layout(a.s, a.dtype);
  if (workspace_bytes < size_t(w.total)) w = bwd_ws_layout(a.s, a.dtype, false);  // as bwd_check
  if (w.total > 0 && !workspace) return fail(SDPA_ERR_WORKSPACE, "backward needs a workspace");
  debug_log("bwd", a, &p.aligned);
  if (a.s.batch == 0 || (a.rows_q == 0 && a.rows_k == 0)) return ok();
  char* ws = static_cast<char*>(workspace);
  p.delta = reinterpret_cast<float*>(ws + w.delta_off);
  p.lse2 = reinterpret_cast<float*>(ws + w.lse2_off);
  p.ws_rows = a.s.thd ? int64_t(a.s.hq) * a.s.total_q : int64_t(a.s.batch) * a.s.hq * a.s.sq;
  p.accumulate = accumulate;
  p.nsplit = 1;
  if (w.split_blocks > 0) {
    p.nsplit = 2;
    p.split_blocks = int32_t(w.split_blocks);
    p.split_cnt = reinterpret_cast<int32_t*>(ws + w.cnt_off);
    p.split_part = reinterpret_cast<float*>(ws + w.part_off);
  }
  if (w.ksplit_cap > 0) {
    p.ksplit_cap = int32_t(w.ksplit_cap);
    p.ksplit_count = reinterpret_cast<int32_t*>(ws + w.kcnt_off);
    p.ksplit_part = reinterpret_cast<float*>(ws + w.kpart_off);
    p.ksplit_cap = bwd_k_split_cap(p, DType(a.dtype));
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (a.s.thd) {
    SchedParams sq = sched_params(a.s, true, reinterpret_cast<WorkItem*>(ws + w.wq_off),
                                  reinterpret_cast<int32_t*>(ws + w.cq_off));
    const bool f32 = a.dtype == SDPA_DTYPE_F32;
    sq.tile_own = bwd_q_tile_rows(p, DType(a.dtype));  // never more items than the workspace holds
    sq.tile_other = f32 ? 32 : kBwdQInner;
    sq.max_items = int32_t(thd_items(a.s.total_q, a.s.batch, sq.tile_own));
    SchedParams sk = sched_params(a.s, false, reinterpret_cast<WorkItem*>(ws + w.wk_off),
                                  reinterpret_cast<int32_t*>(ws + w.ck_off));
    sk.tile_own = bwd_k_tile_rows(p, DType(a.dtype));  // never more items than the workspace holds
    sk.tile_other = f32 ? 32 : kBwdKInner;
    sk.max_items = int32_t(thd_items(a.s.total_k, a.s.batch, sk.tile_own));
    if (p.ksplit_cap > 0) {
      // split the items whose chain of (q head, q tile) steps exceeds the mean per dK/dV
      // workgroup slot (one per CU at head_dim 128, two at 64); a split item takes two entries
      sk.max_items += p.ksplit_cap;
      sk.split_cap = p.ksplit_cap;
      sk.split_heads = a.s.hk;
      sk.split_slots = device_cus() * (a.s.d == 128 ? 1 : 2);
      sk.nsplit = const_cast<int32_t*>(p.ksplit_count);
    }
    if ((e = launch_schedule2(sq, sk, st)) != hipSuccess) return hip_fail(e, "THD schedule launch");
    p.work_q = sq.items;
    p.count_q = sq.count;
    p.work_k = sk.items;
    p.count_k = sk.count;
  }
  if ((e = launch_bwd(p, DType(a.dtype), st)) != hipSuccess) return hip_fail(e, "backward launch");
  return ok();
}

int sdpa_block_mask_build(const sdpa_block_mask_t* mask, int32_t seqlen_q, int32_t seqlen_k,
                          void* stream) {
  if (!mask) return fail(SDPA_ERR_NULL, "mask is NULL");
  if (!mask->bits || !mask->kv_count || !mask->kv_list || !mask->q_count || !mask->q_list)
    return fail(SDPA_ERR_NULL, "block_mask has a NULL array");
  if (mask->batch < 1 || mask->heads < 1 || int64_t(mask->batch) * mask->heads > INT32_MAX)
    return fail(SDPA_ERR_SHAPE, "block_mask batch=%d heads=%d", mask->batch, mask->heads);
  if (seqlen_q < 1 || seqlen_k < 1 || seqlen_q > kMaxSeqlen || seqlen_k > kMaxSeqlen)
    return fail(SDPA_ERR_SHAPE, "seqlen_q=%d seqlen_k=%d", seqlen_q, seqlen_k);
  BmBuildParams bp;
  bp.bits = mask->bits;
  bp.kv_count = mask->kv_count;
  bp.kv_list = mask->kv_list;
  bp.q_count = mask->q_count;
  bp.q_list = mask->q_list;
  bp.planes = int64_t(mask->batch) * mask->heads;
  bp.sq = seqlen_q;
  bp.sk = seqlen_k;
  bp.nqb = (seqlen_q + kMaskBlock - 1) / kMaskBlock;
  bp.nkb = (seqlen_k + kMaskBlock - 1) / kMaskBlock;
  bp.words = (seqlen_k + 63) / 64;
  if (bp.planes * bp.nqb > INT32_MAX || bp.planes * bp.nkb > INT32_MAX)
    return fail(SDPA_ERR_SHAPE, "block_mask too large for one launch");
  hipError_t e = launch_block_mask_build(bp, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "block mask build launch");
  return ok();
}

int sdpa_merge_fwd_validate(const sdpa_merge_desc_t* desc, const sdpa_tensor_t* x_a,
                            const sdpa_rowstat_t* lse_a, const sdpa_tensor_t* x_b,
                            const sdpa_rowstat_t* lse_b, const sdpa_tensor_t* x,
                            const sdpa_rowstat_t* lse) {
  Merge m;
  MergeParams p;
  int rc = merge_fwd_check(desc, x_a, lse_a, x_b, lse_b, x, lse, &m, &p);
  return rc ? rc : ok();
}

int sdpa_merge_bwd_validate(const sdpa_merge_desc_t* desc, const sdpa_tensor_t* x_a,
                            const sdpa_rowstat_t* lse_a, const sdpa_tensor_t* x_b,
                            const sdpa_rowstat_t* lse_b, const sdpa_tensor_t* g,
                            const sdpa_rowstat_t* g_lse, const sdpa_tensor_t* dx_a,
                            const sdpa_rowstat_t* dlse_a, const sdpa_tensor_t* dx_b,
                            const sdpa_rowstat_t* dlse_b) {
  Merge m;
  MergeParams p;
  int rc = merge_bwd_check(desc, x_a, lse_a, x_b, lse_b, g, g_lse, dx_a, dlse_a, dx_b, dlse_b,
                           &m, &p);
  return rc ? rc : ok();
}

int sdpa_merge_fwd(const sdpa_merge_desc_t* desc, const sdpa_tensor_t* x_a,
                   const sdpa_rowstat_t* lse_a, const sdpa_tensor_t* x_b,
                   const sdpa_rowstat_t* lse_b, const sdpa_tensor_t* x,
                   const sdpa_rowstat_t* lse, void* stream) {
  Merge m;
  MergeParams p;
  int rc = merge_fwd_check(desc, x_a, lse_a, x_b, lse_b, x, lse, &m, &p);
  if (rc) return rc;
  if (p.rows == 0) return ok();
  hipError_t e = launch_merge_fwd(p, DType(m.dtype), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "merge forward launch");
  return ok();
}

int sdpa_merge_bwd(const sdpa_merge_desc_t* desc, const sdpa_tensor_t* x_a,
                   const sdpa_rowstat_t* lse_a, const sdpa_tensor_t* x_b,
                   const sdpa_rowstat_t* lse_b, const sdpa_tensor_t* g,
                   const sdpa_rowstat_t* g_lse, const sdpa_tensor_t* dx_a,
                   const sdpa_rowstat_t* dlse_a, const sdpa_tensor_t* dx_b,
                   const sdpa_rowstat_t* dlse_b, void* stream) {
  Merge m;
  MergeParams p;
  int rc = merge_bwd_check(desc, x_a, lse_a, x_b, lse_b, g, g_lse, dx_a, dlse_a, dx_b, dlse_b,
                           &m, &p);
  if (rc) return rc;
  if (p.rows == 0) return ok();
  hipError_t e = launch_merge_bwd(p, DType(m.dtype), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "merge backward launch");
  return ok();
}

}  // extern "C"
