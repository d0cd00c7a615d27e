// Context-parallel ring attention emulated on one GPU ("Add support for cuDNN FusedAttention
// + THD + CP", TransformerEngine issue 885): every sequence is cut into 2 CP chunks and rank
// r holds chunks r and 2 CP - 1 - r (the load-balanced split the page describes); K/V chunk
// pairs travel around a ring, and each rank folds the per-hop partial attentions of its q
// chunks with the LSE merge.  The page states that a ring does not depend on the order of
// its hops; the hop order is an argument here.
//
// Forward, per q chunk i: for every hop, for every kv chunk c the hop brings, the pair
// (i, c) is full (c < i), causal with the diagonal at the chunk start (c == i) or skipped
// (c > i) under a causal mask, and always full without a mask.  The partial (O, LSE) of the
// pair is folded into the running result with sdpa_merge_fwd, in hop order.
// Backward: with the final O and LSE of the whole row, P and Delta of every pair equal those
// of full attention, so each pair's sdpa_bwd adds exactly its share of dQ, dK, dV.  Each
// chunk's diagonal pair writes first (accumulate = 0); every other pair adds in hop order.
//
// THD (the page's own case): chunk c of every sequence at once is a padded-THD view of the
// same tensors (per-sequence row starts and chunk lengths, built on the device by
// launch_cp_chunks; sequences of any length, chunk lengths differing by at most one), and
// the partial results live in full-size packed buffers at the same rows, folded by the merge
// restricted to those rows.
//
// Host orchestration only: every step is an sdpa_fwd / sdpa_merge_fwd / sdpa_bwd launch (and,
// for THD, one launch that builds the chunk views).
#include <stdint.h>
#include <string.h>

#include <string>
#include <vector>

#include <hip/hip_runtime_api.h>

#include "../../include/sdpa.h"
#include "launch.h"

namespace sdpa {
int set_error(int code, const char* msg);
int clear_error();
}  // namespace sdpa

namespace {

constexpr int kMaxCp = 64;

int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// Which logical dimension of a tensor / row statistic is the sequence axis.
int seq_dim(int32_t layout) { return layout == SDPA_LAYOUT_SBHD ? 0 : layout == SDPA_LAYOUT_BSHD ? 1 : 2; }

struct Plan {
  sdpa_desc_t chunk;  // one chunk against one chunk
  int cp = 0, len = 0, esize = 0;
  bool thd = false;
  std::vector<int> order;  // hop h -> ring distance
  int64_t part_x = 0, part_l = 0;  // bytes of a chunk-sized O and LSE (THD: full-size)
  // THD workspace: chunk views, then the fold buffers, then the attention calls' workspace
  int64_t views = 0, attn_off = 0;
  size_t attn_bytes = 0;
};

int plan(const sdpa_desc_t* d, int cp, const int32_t* hop_order, Plan& p) {
  if (!d) return sdpa::set_error(SDPA_ERR_NULL, "descriptor is NULL");
  if (cp < 1 || cp > kMaxCp) return sdpa::set_error(SDPA_ERR_ARG, "cp must be in [1, 64]");
  if (d->layout < 0 || d->layout > SDPA_LAYOUT_THD) return sdpa::set_error(SDPA_ERR_ARG, "bad layout");
  const bool thd = d->layout == SDPA_LAYOUT_THD;
  if (thd && (d->cu_seqlens_q != d->cu_seqlens_k || d->total_q != d->total_k ||
              d->cu_seqlens_q_padded != d->cu_seqlens_k_padded))
    return sdpa::set_error(SDPA_ERR_UNSUPPORTED,
                           "context-parallel THD is self-attention: q and k share cu_seqlens (and padded starts)");
  if (thd && (!d->cu_seqlens_q || d->batch < 0))
    return sdpa::set_error(SDPA_ERR_NULL, "THD needs cu_seqlens");
  if (d->block_mask)
    return sdpa::set_error(SDPA_ERR_UNSUPPORTED, "context-parallel emulation takes no block_mask");
  if (d->seqlen_q != d->seqlen_k)
    return sdpa::set_error(SDPA_ERR_SHAPE, "context-parallel emulation needs seqlen_q == seqlen_k");
  if (!thd && (d->seqlen_q <= 0 || d->seqlen_q % (2 * cp) != 0))
    return sdpa::set_error(SDPA_ERR_SHAPE, "seqlen must be a positive multiple of 2 * cp");
  const bool causal = d->window_left == -1 && d->window_right == 0;
  const bool full = d->window_left == -1 && d->window_right == -1;
  if (!causal && !full)
    return sdpa::set_error(SDPA_ERR_UNSUPPORTED, "context-parallel emulation supports causal (-1,0) or no mask (-1,-1)");
  if (d->dtype == SDPA_DTYPE_FP8_E4M3)
    return sdpa::set_error(SDPA_ERR_UNSUPPORTED, "context-parallel emulation takes fp16, bf16 or fp32");
  p.cp = cp;
  p.thd = thd;
  p.len = thd ? (d->seqlen_q + 2 * cp - 1) / (2 * cp) : d->seqlen_q / (2 * cp);
  p.esize = d->dtype == SDPA_DTYPE_F32 ? 4 : 2;
  p.chunk = *d;
  p.chunk.seqlen_q = p.chunk.seqlen_k = p.len;
  p.chunk.diag_align = SDPA_ALIGN_TOP_LEFT;
  p.order.resize(cp);
  std::vector<char> seen(cp, 0);
  for (int h = 0; h < cp; ++h) {
    const int v = hop_order ? hop_order[h] : h;
    if (v < 0 || v >= cp || seen[v]) return sdpa::set_error(SDPA_ERR_ARG, "hop_order must be a permutation of 0..cp-1");
    seen[v] = 1;
    p.order[h] = v;
  }
  if (thd) {
    p.part_x = d->total_q * d->heads_q * d->head_dim * p.esize;
    p.part_l = d->total_q * d->heads_q * 4;
    p.views = round_up(int64_t(2 * cp) * 2 * (d->batch + 1) * 4, 256);
    size_t fw = 0, bw = 0;
    int rc;
    if ((rc = sdpa_fwd_workspace_size(&p.chunk, &fw)) || (rc = sdpa_bwd_workspace_size(&p.chunk, &bw))) return rc;
    p.attn_bytes = fw > bw ? fw : bw;
    p.attn_off = p.views + 3 * (round_up(p.part_x, 256) + round_up(p.part_l, 256));
  } else {
    p.part_x = int64_t(d->batch) * d->heads_q * p.len * d->head_dim * p.esize;
    p.part_l = int64_t(d->batch) * d->heads_q * p.len * 4;
  }
  return SDPA_OK;
}

// THD: chunk c's view arrays in the workspace (row starts, then the prefix of lengths)
const int32_t* view_starts(const Plan& p, void* ws, int c) {
  return static_cast<const int32_t*>(ws) + int64_t(c) * 2 * (p.chunk.batch + 1);
}
const int32_t* view_prefix(const Plan& p, void* ws, int c) {
  return view_starts(p, ws, c) + (p.chunk.batch + 1);
}
// The descriptor of pair (q chunk i, kv chunk c) for THD
sdpa_desc_t thd_pair(const Plan& p, void* ws, int i, int c) {
  sdpa_desc_t cd = p.chunk;
  cd.cu_seqlens_q = view_prefix(p, ws, i);
  cd.cu_seqlens_q_padded = view_starts(p, ws, i);
  cd.cu_seqlens_k = view_prefix(p, ws, c);
  cd.cu_seqlens_k_padded = view_starts(p, ws, c);
  return cd;
}

bool causal_of(const sdpa_desc_t* d) { return d->window_right == 0; }

// Chunk c of a full-sequence tensor / row statistic: same strides, base moved along s.
sdpa_tensor_t chunk_of(const sdpa_tensor_t& t, int32_t layout, int c, int len, int esize) {
  sdpa_tensor_t r = t;
  r.data = static_cast<char*>(t.data) + int64_t(c) * len * t.stride[seq_dim(layout)] * esize;
  return r;
}
sdpa_rowstat_t chunk_of(const sdpa_rowstat_t& t, int c, int len) {
  sdpa_rowstat_t r = t;
  if (t.data) r.data = t.data + int64_t(c) * len * t.stride[2];
  return r;
}

// A contiguous chunk-sized tensor / row statistic in the layout's logical order.
sdpa_tensor_t dense(void* base, const sdpa_desc_t& c) {
  sdpa_tensor_t t;
  t.data = base;
  const int64_t b = c.batch, s = c.seqlen_q, h = c.heads_q, d = c.head_dim;
  if (c.layout == SDPA_LAYOUT_BSHD) { t.stride[0] = s * h * d; t.stride[1] = h * d; t.stride[2] = d; }
  else if (c.layout == SDPA_LAYOUT_SBHD) { t.stride[0] = b * h * d; t.stride[1] = h * d; t.stride[2] = d; }
  else { t.stride[0] = h * s * d; t.stride[1] = s * d; t.stride[2] = d; }
  t.stride[3] = 1;
  return t;
}
sdpa_rowstat_t dense_stat(void* base, const sdpa_desc_t& c) {
  sdpa_rowstat_t t;
  t.data = static_cast<float*>(base);
  t.stride[0] = int64_t(c.heads_q) * c.seqlen_q;
  t.stride[1] = c.seqlen_q;
  t.stride[2] = 1;
  return t;
}

// The chunks rank r holds, and the window of pair (i, c); false when the pair is skipped.
void chunks_of(int r, int cp, int out[2]) {
  out[0] = r;
  out[1] = 2 * cp - 1 - r;
}
bool pair_window(bool causal, int i, int c, int32_t& left, int32_t& right) {
  left = -1;
  right = -1;
  if (!causal) return true;
  if (c > i) return false;
  if (c == i) right = 0;
  return true;
}

}  // namespace

extern "C" {

int sdpa_cp_workspace_size(const sdpa_desc_t* desc, int cp, size_t* bytes) {
  Plan p;
  int rc = plan(desc, cp, nullptr, p);
  if (rc) return rc;
  if (!bytes) return sdpa::set_error(SDPA_ERR_NULL, "bytes is NULL");
  if (p.thd) {
    *bytes = size_t(p.attn_off) + p.attn_bytes;
    return sdpa::clear_error();
  }
  size_t bw = 0;
  if ((rc = sdpa_bwd_workspace_size(&p.chunk, &bw))) return rc;
  const int64_t fold = 3 * (round_up(p.part_x, 256) + round_up(p.part_l, 256));
  *bytes = size_t(fold > int64_t(bw) ? fold : int64_t(bw));
  return sdpa::clear_error();
}

int sdpa_cp_fwd(const sdpa_desc_t* desc, int cp, const int32_t* hop_order, const sdpa_tensor_t* q,
                const sdpa_tensor_t* k, const sdpa_tensor_t* v, const sdpa_tensor_t* o,
                const sdpa_rowstat_t* lse, void* workspace, size_t workspace_bytes, void* stream) {
  Plan p;
  int rc = plan(desc, cp, hop_order, p);
  if (rc) return rc;
  if ((rc = sdpa_fwd_validate(desc, q, k, v, o, lse, SIZE_MAX))) return rc;
  if (!lse || !lse->data) return sdpa::set_error(SDPA_ERR_NULL, "context-parallel forward needs the LSE output");
  size_t need = 0;
  if ((rc = sdpa_cp_workspace_size(desc, cp, &need))) return rc;
  if (!workspace || workspace_bytes < need) return sdpa::set_error(SDPA_ERR_WORKSPACE, "workspace missing or too small");

  // workspace: (THD: the chunk views, then) partial (x, lse) and two running results, used
  // in turn (THD: full-size packed buffers, then the attention calls' own workspace)
  char* ws = static_cast<char*>(workspace);
  const int64_t xs = round_up(p.part_x, 256), ls = round_up(p.part_l, 256);
  sdpa_tensor_t bx[3];
  sdpa_rowstat_t bl[3];
  for (int i = 0; i < 3; ++i) {
    char* b = ws + p.views + i * (xs + ls);
    if (p.thd) {
      const int64_t h = desc->heads_q, d = desc->head_dim;
      bx[i] = sdpa_tensor_t{b, {h * d, d, 1, 0}};
      bl[i] = sdpa_rowstat_t{reinterpret_cast<float*>(b + xs), {desc->total_q, 1, 0}};
    } else {
      bx[i] = dense(b, p.chunk);
      bl[i] = dense_stat(b + xs, p.chunk);
    }
  }
  void* attn_ws = p.thd ? ws + p.attn_off : nullptr;
  const size_t attn_bytes = p.thd ? p.attn_bytes : 0;
  if (p.thd) {
    if (hipError_t e = sdpa::launch_cp_chunks(desc->cu_seqlens_q, desc->cu_seqlens_q_padded, desc->batch,
                                              desc->total_q, cp, reinterpret_cast<int32_t*>(ws),
                                              static_cast<hipStream_t>(stream)))
      return sdpa::set_error(SDPA_ERR_HIP, hipGetErrorString(e));
  }
  sdpa_merge_desc_t md{desc->layout, desc->dtype, desc->batch, p.len, desc->heads_q, desc->head_dim,
                       p.thd ? desc->total_q : 0, nullptr, nullptr};
  const bool causal = causal_of(desc);
  const int L = p.len, es = p.esize;
  for (int r = 0; r < cp; ++r) {
    int mine[2];
    chunks_of(r, cp, mine);
    for (int qi = 0; qi < 2; ++qi) {
      const int i = mine[qi];
      // the pairs of q chunk i, in hop order
      std::vector<int> kvs;
      for (int h = 0; h < cp; ++h) {
        int src[2];
        chunks_of(((r - p.order[h]) % cp + cp) % cp, cp, src);
        for (int c : {src[0] < src[1] ? src[0] : src[1], src[0] < src[1] ? src[1] : src[0]}) {
          int32_t wl, wr;
          if (pair_window(causal, i, c, wl, wr)) kvs.push_back(c);
        }
      }
      // dense: chunk views; THD: the whole tensors, rows picked by the chunk views
      const sdpa_tensor_t qc = p.thd ? *q : chunk_of(*q, desc->layout, i, L, es);
      const sdpa_tensor_t oc = p.thd ? *o : chunk_of(*o, desc->layout, i, L, es);
      const sdpa_rowstat_t lc = p.thd ? *lse : chunk_of(*lse, i, L);
      if (p.thd) {
        md.cu_seqlens = view_prefix(p, ws, i);
        md.cu_seqlens_padded = view_starts(p, ws, i);
      }
      int run = -1;  // which buffer holds the running result
      for (size_t n = 0; n < kvs.size(); ++n) {
        const int c = kvs[n];
        sdpa_desc_t cd = p.thd ? thd_pair(p, ws, i, c) : p.chunk;
        pair_window(causal, i, c, cd.window_left, cd.window_right);
        const sdpa_tensor_t kc = p.thd ? *k : chunk_of(*k, desc->layout, c, L, es);
        const sdpa_tensor_t vc = p.thd ? *v : chunk_of(*v, desc->layout, c, L, es);
        const bool last = n + 1 == kvs.size();
        if (n == 0) {  // first partial: straight into the running buffer (or the output)
          const sdpa_tensor_t& ox = last ? oc : bx[1];
          const sdpa_rowstat_t& ol = last ? lc : bl[1];
          if ((rc = sdpa_fwd(&cd, &qc, &kc, &vc, &ox, &ol, attn_ws, attn_bytes, stream))) return rc;
          run = 1;
          continue;
        }
        if ((rc = sdpa_fwd(&cd, &qc, &kc, &vc, &bx[0], &bl[0], attn_ws, attn_bytes, stream))) return rc;
        const int nxt = run == 1 ? 2 : 1;
        const sdpa_tensor_t& ox = last ? oc : bx[nxt];
        const sdpa_rowstat_t& ol = last ? lc : bl[nxt];
        if ((rc = sdpa_merge_fwd(&md, &bx[run], &bl[run], &bx[0], &bl[0], &ox, &ol, stream))) return rc;
        run = nxt;
      }
    }
  }
  return sdpa::clear_error();
}

int sdpa_cp_bwd(const sdpa_desc_t* desc, int cp, const int32_t* hop_order, const sdpa_tensor_t* q,
                const sdpa_tensor_t* k, const sdpa_tensor_t* v, const sdpa_tensor_t* o,
                const sdpa_rowstat_t* lse, const sdpa_tensor_t* dout, const sdpa_rowstat_t* dlse,
                const sdpa_tensor_t* dq, const sdpa_tensor_t* dk, const sdpa_tensor_t* dv,
                void* workspace, size_t workspace_bytes, void* stream) {
  Plan p;
  int rc = plan(desc, cp, hop_order, p);
  if (rc) return rc;
  // tensors of the whole problem (its own workspace is not used: each pair brings its own)
  if ((rc = sdpa_bwd_validate(desc, q, k, v, o, lse, dout, dlse, dq, dk, dv, SIZE_MAX))) return rc;
  size_t need = 0;
  if ((rc = sdpa_cp_workspace_size(desc, cp, &need))) return rc;
  if (!workspace || workspace_bytes < need) return sdpa::set_error(SDPA_ERR_WORKSPACE, "workspace missing or too small");
  const bool causal = causal_of(desc);
  const int L = p.len, es = p.esize;
  const bool has_dlse = dlse && dlse->data;
  char* ws = static_cast<char*>(workspace);
  if (p.thd) {
    if (hipError_t e = sdpa::launch_cp_chunks(desc->cu_seqlens_q, desc->cu_seqlens_q_padded, desc->batch,
                                              desc->total_q, cp, reinterpret_cast<int32_t*>(ws),
                                              static_cast<hipStream_t>(stream)))
      return sdpa::set_error(SDPA_ERR_HIP, hipGetErrorString(e));
  }
  auto pair = [&](int i, int c, int accumulate) {
    const sdpa_rowstat_t nodl{nullptr, {0, 0, 0}};
    if (p.thd) {  // whole tensors, rows picked by the chunk views
      sdpa_desc_t cd = thd_pair(p, ws, i, c);
      pair_window(causal, i, c, cd.window_left, cd.window_right);
      return sdpa_bwd(&cd, q, k, v, o, lse, dout, has_dlse ? dlse : &nodl, dq, dk, dv, accumulate,
                      ws + p.attn_off, p.attn_bytes, stream);
    }
    sdpa_desc_t cd = p.chunk;
    pair_window(causal, i, c, cd.window_left, cd.window_right);
    const sdpa_tensor_t qc = chunk_of(*q, desc->layout, i, L, es), oc = chunk_of(*o, desc->layout, i, L, es);
    const sdpa_tensor_t gc = chunk_of(*dout, desc->layout, i, L, es), dqc = chunk_of(*dq, desc->layout, i, L, es);
    const sdpa_tensor_t kc = chunk_of(*k, desc->layout, c, L, es), vc = chunk_of(*v, desc->layout, c, L, es);
    const sdpa_tensor_t dkc = chunk_of(*dk, desc->layout, c, L, es), dvc = chunk_of(*dv, desc->layout, c, L, es);
    const sdpa_rowstat_t lc = chunk_of(*lse, i, L);
    const sdpa_rowstat_t dlc = has_dlse ? chunk_of(*dlse, i, L) : nodl;
    return sdpa_bwd(&cd, &qc, &kc, &vc, &oc, &lc, &gc, &dlc, &dqc, &dkc, &dvc, accumulate, workspace,
                    workspace_bytes, stream);
  };
  // every chunk's diagonal pair initialises its dq, dk, dv
  for (int c = 0; c < 2 * cp; ++c)
    if ((rc = pair(c, c, 0))) return rc;
  // the rest, rank by rank in hop order
  for (int r = 0; r < cp; ++r) {
    int mine[2];
    chunks_of(r, cp, mine);
    for (int h = 0; h < cp; ++h) {
      int src[2];
      chunks_of(((r - p.order[h]) % cp + cp) % cp, cp, src);
      for (int qi = 0; qi < 2; ++qi)
        for (int c : src) {
          const int i = mine[qi];
          int32_t wl, wr;
          if (c == i || !pair_window(causal, i, c, wl, wr)) continue;
          if ((rc = pair(i, c, 1))) return rc;
        }
    }
  }
  return sdpa::clear_error();
}

}  // extern "C"
