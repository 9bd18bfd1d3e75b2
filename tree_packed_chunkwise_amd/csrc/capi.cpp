// capi.cpp -- extern "C" entry points of libkda_tree.so (declared in include/kda_tree.h).
//
// Argument checking, buffer carving and launch sequencing only; every step of
// the computation runs in the HIP kernels (kda_prep.hip, kda_fwd.hip,
// kda_bwd.hip, kda_grad.hip, kda_reduce.hip, attn.hip, gather.hip), enqueued
// on the caller's stream (the forward and reverse calls also fork a second
// stream of the device and join it back before returning: schedule.cpp).
#include <initializer_list>
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <string>

#include "kda_tree.h"
#include "common.h"
#include "plan.h"

namespace kda {
hipError_t run_fwd(const FwdArgs& a, bool bf16, int BC, int D, const Plan& p, hipStream_t st);
hipError_t run_bwd(const BwdArgs& a, bool bf16, int BC, int D, const Plan& p, hipStream_t st);
void set_overlap(bool on);
hipError_t launch_attn_fwd(const AttnArgs& a, int D, int n_tiles, hipStream_t st);
hipError_t launch_attn_bwd(const AttnArgs& a, int D, int64_t n_rows, int n_tiles, int n_items,
                           int n_split, hipStream_t st);
hipError_t launch_gather_fwd(const void* logits, bool bf16, int64_t n_rows, int vocab,
                             const int* pos_row, const int* pos_tgt, int64_t n_pos, float* logp,
                             float* lse, hipStream_t st);
hipError_t launch_gather_bwd(const void* logits, bool bf16, int64_t n_rows, int vocab,
                             const float* lse, const int* row_pos_ptr, const int* row_pos_idx,
                             const int* pos_tgt, const float* dlogp, void* dlogits,
                             hipStream_t st);
size_t router_ws_bytes(int64_t n_rows, int E);
hipError_t launch_router_stats(const void* x, bool bf16, int64_t n_rows, int E, int k,
                               const int* q, int* tidx, float* tprob, int64_t* load, float* psum,
                               float* zsum, int64_t* n_tok, void* ws, hipStream_t st);
hipError_t launch_router_bwd(const void* x, bool bf16, int64_t n_rows, int E, const int* q,
                             const float* g, float gz, float* dx, hipStream_t st);
hipError_t router_scratch(void** ptr, size_t* bytes);
int l1_plan(int32_t n, const int32_t* parent, const int32_t* seg_len, int64_t budget,
            std::vector<int32_t>& leaf_mb, std::vector<int64_t>& mb_unique,
            std::vector<int64_t>& mb_expanded, std::string& err);
hipError_t launch_state_copy(const float* src, const int* sidx, float* dst, const int* didx, int n,
                             int64_t elems, hipStream_t st);
hipError_t launch_state_sum(const float* src, const int* ptr, const int* idx, int n_dst,
                            int64_t elems, int accumulate, float* dst, hipStream_t st);
}  // namespace kda

struct kda_plan {
  kda::Plan p;
};

namespace {

thread_local std::string g_err;

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

int hip_fail(hipError_t e, const char* where) {
  return fail(KDA_ERR_HIP, std::string(where) + ": " + hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
inline size_t al(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Carves consecutive 256-byte-aligned float regions out of a byte buffer.
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base((char*)b) {}
  float* take(size_t nfloats) {
    float* p = base ? (float*)(base + off) : nullptr;
    off += al(nfloats * sizeof(float));
    return p;
  }
};

bool shape_ok(int32_t B, int32_t H, int32_t dk, int32_t dv) {
  return H > 0 && dk == dv && (dk == 64 || dk == 128) && (B == 16 || B == 64);
}

kda::DevPlan make_dev_plan(const kda::Plan& p, const void* dev) {
  const int32_t* b = (const int32_t*)dev;
  const kda::DevLayout& d = p.dev;
  kda::DevPlan v;
  v.round_seq_ptr = b + d.round_seq_ptr;
  v.seq_chunk_ptr = b + d.seq_chunk_ptr;
  v.seq_row_ptr = b + d.seq_row_ptr;
  v.seq_init_kind = b + d.seq_init_kind;
  v.seq_init_idx = b + d.seq_init_idx;
  v.seq_leaf = b + d.seq_leaf;
  v.seq_lpt = b + d.seq_lpt;
  v.chunk_seq = b + d.chunk_seq;
  v.chunk_row0 = b + d.chunk_row0;
  v.chunk_len = b + d.chunk_len;
  v.chunk_save = b + d.chunk_save;
  v.chunk_nrep = b + d.chunk_nrep;
  v.chunk_rep0 = b + d.chunk_rep0;
  v.chunk_round = b + d.chunk_round;
  v.row_index = b + d.row_index;
  v.out_row = b + d.out_row;
  v.buf_cons_ptr = b + d.buf_cons_ptr;
  v.buf_cons = b + d.buf_cons;
  v.buf_chunk = b + d.buf_chunk;
  v.rep_row = b + d.rep_row;
  v.rep_ptr = b + d.rep_ptr;
  v.rep_slot = b + d.rep_slot;
  v.root_seq_ptr = b + d.root_seq_ptr;
  v.root_seq = b + d.root_seq;
  return v;
}

// saved = [chunk start states (fp16) | handoff states | chunk images]
//         (image layout in chunk.h; the image reserves fp32 space for V
//         whatever the input dtype)
struct SavedView {
  _Float16* chunk_h;
  float* bufs;
  unsigned char* fimg;
};
SavedView carve_saved(const kda::Plan& p, int H, int D, void* base, size_t* total) {
  Carver c(base);
  SavedView s;
  const size_t st = (size_t)H * D * D;
  s.chunk_h = (_Float16*)c.take((size_t)p.n_chunks() * st / 2);
  s.bufs = c.take((size_t)p.n_buf() * st);
  const size_t nb = (size_t)p.n_chunks() * H;
  s.fimg = (unsigned char*)c.take(nb * kda::fwd_image_bytes(p.B, D) / 4);
  if (total) *total = c.off;
  return s;
}

// bwd workspace = [dO tiles per chunk-head (sized for fp32) | dy tiles | chunk
//                  end-state gradients (fp16) | sequence start gradients |
//                  replay-row gradients | gradient-scale words (common.h)]
struct BwdWS {
  float *dOp, *slot, *rep_dq, *rep_dk, *rep_dg, *rep_dv, *rep_db;
  _Float16 *dy, *dhc;
  unsigned* gmax;
};
BwdWS carve_bwd_ws(const kda::Plan& p, int H, int D, void* base, size_t* total) {
  Carver c(base);
  BwdWS w;
  const size_t nb = (size_t)p.n_chunks() * H;
  w.dOp = c.take(nb * p.B * D);  // per chunk-head 16x16 tiles
  w.dy = (_Float16*)c.take(nb * p.B * D / 2);   // fp16, per chunk-head 16x16 tiles
  w.dhc = (_Float16*)c.take(nb * D * D / 2);
  w.slot = c.take((size_t)p.n_seq() * H * D * D);
  const size_t nrep = (size_t)p.R;
  w.rep_dq = c.take(nrep * H * D);
  w.rep_dk = c.take(nrep * H * D);
  w.rep_dg = c.take(nrep * H * D);
  w.rep_dv = c.take(nrep * H * D);
  w.rep_db = c.take(nrep * H);
  w.gmax = (unsigned*)c.take(kda::scale_words(p.n_rounds));
  if (total) *total = c.off;
  return w;
}

// kernels move tensor rows in 16-byte vectors
bool aligned16(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (((uintptr_t)p) % 16) return false;
  return true;
}

int check_dev_plan(const kda_plan* plan, const void* dev_plan) {
  if (!plan) return fail(KDA_ERR_ARG, "plan is null");
  if (!dev_plan) return fail(KDA_ERR_ARG, "dev_plan is null");
  if (((uintptr_t)dev_plan) % 4) return fail(KDA_ERR_ARG, "dev_plan misaligned");
  return KDA_OK;
}

}  // namespace

extern "C" {

const char* kda_last_error(void) { return g_err.c_str(); }

int kda_tree_plan(int32_t n_seg, const int32_t* parent, const int32_t* seg_len,
                  const int64_t* seg_row, int32_t chunk, int32_t mode, kda_plan** out) {
  if (!out) return fail(KDA_ERR_ARG, "out is null");
  *out = nullptr;
  kda_plan* p = new kda_plan();
  std::string err;
  int rc = kda::build_plan(n_seg, parent, seg_len, seg_row, chunk, mode, p->p, err);
  if (rc != 0) {
    delete p;
    return fail(rc, err);
  }
  *out = p;
  g_err.clear();
  return KDA_OK;
}

void kda_plan_destroy(kda_plan* plan) { delete plan; }

int kda_l1_plan(int32_t n_seg, const int32_t* parent, const int32_t* seg_len, int64_t budget,
                int32_t* leaf_mb, int32_t* n_mb, int64_t* mb_unique, int64_t* mb_expanded) {
  if (!parent || !seg_len || !leaf_mb || !n_mb || !mb_unique || !mb_expanded)
    return fail(KDA_ERR_ARG, "null argument");
  std::vector<int32_t> lm;
  std::vector<int64_t> mu, mx;
  std::string err;
  if (kda::l1_plan(n_seg, parent, seg_len, budget, lm, mu, mx, err) != 0)
    return fail(KDA_ERR_TREE, err);
  std::copy(lm.begin(), lm.end(), leaf_mb);
  std::copy(mu.begin(), mu.end(), mb_unique);
  std::copy(mx.begin(), mx.end(), mb_expanded);
  *n_mb = (int32_t)mu.size();
  g_err.clear();
  return KDA_OK;
}

int kda_plan_info(const kda_plan* plan, kda_plan_info_t* info) {
  if (!plan || !info) return fail(KDA_ERR_ARG, "null argument");
  const kda::Plan& p = plan->p;
  std::memset(info, 0, sizeof(*info));
  info->n_seg = p.n_seg;
  info->n_rounds = p.n_rounds;
  info->n_seq = p.n_seq();
  info->n_chunks = p.n_chunks();
  info->n_buf = p.n_buf();
  info->n_leaf = p.n_leaf;
  info->n_root = p.n_root;
  info->chunk = p.B;
  info->mode = p.mode;
  info->max_seq_per_round = p.max_seq_per_round;
  info->n_rows = p.n_rows;
  info->n_packed = p.n_packed;
  info->n_out_rows = p.n_out_rows;
  info->R = p.R;
  info->n_pos = (int64_t)p.pos_row.size();
  info->n_expanded = p.n_expanded;
  info->device_bytes = (size_t)p.dev.total * sizeof(int32_t);
  info->n_att_tiles = (int32_t)p.att_tile_seg.size();
  info->n_att_items = (int32_t)p.att_kw_tile.size();
  info->n_att_slots = p.att_n_slots;
  info->n_att_split = (int32_t)p.att_ks_tile.size();
  return KDA_OK;
}

int64_t kda_plan_export(const kda_plan* plan, int32_t field, int64_t* dst, int64_t n) {
  if (!plan) return fail(KDA_ERR_ARG, "plan is null");
  const kda::Plan& p = plan->p;
  auto put32 = [&](const std::vector<int32_t>& v) -> int64_t {
    const int64_t len = (int64_t)v.size();
    if (dst) {
      if (n < len) return fail(KDA_ERR_ARG, "export buffer too small");
      for (int64_t i = 0; i < len; ++i) dst[i] = v[i];
    }
    return len;
  };
  auto put64 = [&](const std::vector<int64_t>& v) -> int64_t {
    const int64_t len = (int64_t)v.size();
    if (dst) {
      if (n < len) return fail(KDA_ERR_ARG, "export buffer too small");
      for (int64_t i = 0; i < len; ++i) dst[i] = v[i];
    }
    return len;
  };
  switch (field) {
    case KDA_F_SEG_ROUND: return put32(p.seg_round);
    case KDA_F_SEG_SEQ: return put32(p.seg_seq);
    case KDA_F_SEG_IS_CONT: return put32(p.seg_is_cont);
    case KDA_F_SEG_B: return put32(p.seg_b);
    case KDA_F_SEG_REPLAY: return put32(p.seg_replay);
    case KDA_F_ROUND_SEQ_PTR: return put32(p.round_seq_ptr);
    case KDA_F_SEQ_ROUND: return put32(p.seq_round);
    case KDA_F_SEQ_HEAD: return put32(p.seq_head);
    case KDA_F_SEQ_LEAF: return put32(p.seq_leaf);
    case KDA_F_SEQ_B_HEAD: return put32(p.seq_b_head);
    case KDA_F_SEQ_REPLAY: return put32(p.seq_replay);
    case KDA_F_SEQ_ROW_PTR: return put32(p.seq_row_ptr);
    case KDA_F_SEQ_CHUNK_PTR: return put32(p.seq_chunk_ptr);
    case KDA_F_SEQ_INIT_KIND: return put32(p.seq_init_kind);
    case KDA_F_SEQ_INIT_IDX: return put32(p.seq_init_idx);
    case KDA_F_CHUNK_SEQ: return put32(p.chunk_seq);
    case KDA_F_CHUNK_ROW0: return put32(p.chunk_row0);
    case KDA_F_CHUNK_LEN: return put32(p.chunk_len);
    case KDA_F_CHUNK_SAVE: return put32(p.chunk_save);
    case KDA_F_ROW_INDEX: return put32(p.row_index);
    case KDA_F_OUT_ROW: return put32(p.out_row);
    case KDA_F_BUF_SEQ: return put32(p.buf_seq);
    case KDA_F_BUF_POS: return put64(p.buf_pos);
    case KDA_F_BUF_CHUNK: return put32(p.buf_chunk);
    case KDA_F_BUF_CONS_PTR: return put32(p.buf_cons_ptr);
    case KDA_F_BUF_CONS: return put32(p.buf_cons);
    case KDA_F_POS_ROW: return put32(p.pos_row);
    case KDA_F_POS_NEXT_ROW: return put32(p.pos_next_row);
    case KDA_F_ROW_POS_PTR: return put32(p.row_pos_ptr);
    case KDA_F_ROW_POS_IDX: return put32(p.row_pos_idx);
    case KDA_F_LEAF_SEG: return put32(p.leaf_seg);
    case KDA_F_ROOT_SEG: return put32(p.root_seg);
    case KDA_F_ATT_ANC_PTR: return put32(p.att_anc_ptr);
    case KDA_F_ATT_ANC: return put32(p.att_anc);
    case KDA_F_ATT_SEG_TILE0: return put32(p.att_seg_tile0);
    case KDA_F_ATT_TILE_SEG: return put32(p.att_tile_seg);
    case KDA_F_ATT_TILE_OFF: return put32(p.att_tile_off);
    case KDA_F_ATT_QORDER: return put32(p.att_qorder);
    case KDA_F_ATT_KQ_PTR: return put32(p.att_kq_ptr);
    case KDA_F_ATT_KQ: return put32(p.att_kq);
    case KDA_F_ATT_KW_TILE: return put32(p.att_kw_tile);
    case KDA_F_ATT_KW_Q0: return put32(p.att_kw_q0);
    case KDA_F_ATT_KW_NQ: return put32(p.att_kw_nq);
    case KDA_F_ATT_KW_SLOT: return put32(p.att_kw_slot);
    case KDA_F_ROW_MULT: return put32(p.row_mult);
    case KDA_F_SEQ_LPT: return put32(p.seq_lpt);
    default: return fail(KDA_ERR_ARG, "unknown export field");
  }
}

int kda_plan_upload(const kda_plan* plan, void* dev, size_t bytes, void* stream) {
  if (!plan || !dev) return fail(KDA_ERR_ARG, "null argument");
  const kda::Plan& p = plan->p;
  const size_t need = (size_t)p.dev.total * sizeof(int32_t);
  if (bytes < need) return fail(KDA_ERR_WORKSPACE, "device plan buffer too small");
  if (((uintptr_t)dev) % 256) return fail(KDA_ERR_ARG, "device plan buffer must be 256-byte aligned");
  hipError_t e = hipMemcpyAsync(dev, p.dev_blob.data(), need, hipMemcpyHostToDevice,
                                (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "kda_plan_upload");
  return KDA_OK;
}

int64_t kda_plan_device_offset(const kda_plan* plan, int32_t field) {
  if (!plan) return fail(KDA_ERR_ARG, "plan is null");
  const kda::DevLayout& d = plan->p.dev;
  switch (field) {
    case KDA_F_POS_ROW: return d.pos_row * 4;
    case KDA_F_POS_NEXT_ROW: return d.pos_next_row * 4;
    case KDA_F_ROW_POS_PTR: return d.row_pos_ptr * 4;
    case KDA_F_ROW_POS_IDX: return d.row_pos_idx * 4;
    case KDA_F_ROW_INDEX: return d.row_index * 4;
    case KDA_F_OUT_ROW: return d.out_row * 4;
    case KDA_F_ROW_MULT: return d.row_mult * 4;
    default: return fail(KDA_ERR_ARG, "field has no device table");
  }
}

size_t kda_saved_bytes(const kda_plan* plan, int32_t H, int32_t dk, int32_t dv) {
  if (!plan || !shape_ok(plan->p.B, H, dk, dv)) return 0;
  size_t total = 0;
  carve_saved(plan->p, H, dk, nullptr, &total);
  return total;
}

size_t kda_fwd_workspace_bytes(const kda_plan* plan, int32_t H, int32_t dk, int32_t dv) {
  if (!plan || !shape_ok(plan->p.B, H, dk, dv)) return 0;
  return kAlign;  // the forward keeps everything it needs in `saved`
}

size_t kda_bwd_workspace_bytes(const kda_plan* plan, int32_t H, int32_t dk, int32_t dv) {
  if (!plan || !shape_ok(plan->p.B, H, dk, dv)) return 0;
  size_t total = 0;
  carve_bwd_ws(plan->p, H, dk, nullptr, &total);
  return total;
}

int kda_tree_fwd(const kda_plan* plan, const void* dev_plan, int32_t H, int32_t dk, int32_t dv,
                 int32_t in_dtype, float scale, const void* q, const void* k, const void* v,
                 const float* g, const float* beta, const float* h0, float* o, float* h_leaf,
                 void* saved, size_t saved_bytes, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_dev_plan(plan, dev_plan);
  if (rc) return rc;
  const kda::Plan& p = plan->p;
  if (!shape_ok(p.B, H, dk, dv))
    return fail(KDA_ERR_SHAPE, "supported: dk == dv in {64,128}, chunk in {16,64}, H > 0");
  if (in_dtype != KDA_DTYPE_BF16 && in_dtype != KDA_DTYPE_FP32)
    return fail(KDA_ERR_SHAPE, "in_dtype must be KDA_DTYPE_BF16 or KDA_DTYPE_FP32");
  if (!q || !k || !v || !g || !beta || !o || !h_leaf || !saved || !ws)
    return fail(KDA_ERR_ARG, "null tensor argument");
  if (!aligned16({q, k, v, g, h0, o, h_leaf, saved, ws}) || ((uintptr_t)beta) % 4)
    return fail(KDA_ERR_ARG, "tensor arguments must be 16-byte aligned (beta: 4-byte)");
  if (saved_bytes < kda_saved_bytes(plan, H, dk, dv))
    return fail(KDA_ERR_WORKSPACE, "saved buffer too small");
  if (ws_bytes < kda_fwd_workspace_bytes(plan, H, dk, dv))
    return fail(KDA_ERR_WORKSPACE, "forward workspace too small");
  kda::FwdArgs a;
  a.plan = make_dev_plan(p, dev_plan);
  a.H = H;
  a.scale = scale;
  a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.h0 = h0;
  a.o = o;
  a.h_leaf = h_leaf;
  SavedView sv = carve_saved(p, H, dk, saved, nullptr);
  a.chunk_h = sv.chunk_h;
  a.bufs = sv.bufs;
  a.fimg = sv.fimg;
  hipError_t e = kda::run_fwd(a, in_dtype == KDA_DTYPE_BF16, p.B, dk, p, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "kda_tree_fwd launch");
  return KDA_OK;
}

int kda_tree_bwd(const kda_plan* plan, const void* dev_plan, int32_t H, int32_t dk, int32_t dv,
                 int32_t in_dtype, float scale, const void* q, const void* k, const void* v,
                 const float* g, const float* beta, const float* h0, const void* saved,
                 size_t saved_bytes, const void* dO, const float* dh_leaf, float* dq, float* dk_,
                 float* dv_, float* dg, float* dbeta, float* dh0, float* dh_boundary, void* ws,
                 size_t ws_bytes, void* stream) {
  (void)h0;  // the start states of all chunks are in `saved`
  int rc = check_dev_plan(plan, dev_plan);
  if (rc) return rc;
  const kda::Plan& p = plan->p;
  if (!shape_ok(p.B, H, dk, dv))
    return fail(KDA_ERR_SHAPE, "supported: dk == dv in {64,128}, chunk in {16,64}, H > 0");
  if (in_dtype != KDA_DTYPE_BF16 && in_dtype != KDA_DTYPE_FP32)
    return fail(KDA_ERR_SHAPE, "in_dtype must be KDA_DTYPE_BF16 or KDA_DTYPE_FP32");
  if (!q || !k || !v || !g || !beta || !saved || !dO || !dq || !dk_ || !dv_ || !dg || !dbeta ||
      !dh0 || !ws)
    return fail(KDA_ERR_ARG, "null tensor argument");
  if (!aligned16({q, k, v, g, saved, dO, dh_leaf, dq, dk_, dv_, dg, dh0, dh_boundary, ws}) ||
      ((uintptr_t)beta) % 4 || ((uintptr_t)dbeta) % 4)
    return fail(KDA_ERR_ARG, "tensor arguments must be 16-byte aligned (beta, dbeta: 4-byte)");
  if (saved_bytes < kda_saved_bytes(plan, H, dk, dv))
    return fail(KDA_ERR_WORKSPACE, "saved buffer too small");
  if (ws_bytes < kda_bwd_workspace_bytes(plan, H, dk, dv))
    return fail(KDA_ERR_WORKSPACE, "backward workspace too small");
  SavedView sv = carve_saved(p, H, dk, (void*)saved, nullptr);
  BwdWS w = carve_bwd_ws(p, H, dk, ws, nullptr);
  kda::BwdArgs a;
  a.plan = make_dev_plan(p, dev_plan);
  a.H = H;
  a.scale = scale;
  a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
  a.chunk_h = sv.chunk_h;
  a.fimg = sv.fimg;
  a.dO = dO;
  a.dh_leaf = dh_leaf;
  a.dq = dq; a.dk = dk_; a.dv = dv_; a.dg = dg; a.dbeta = dbeta; a.dh0 = dh0;
  a.dh_boundary = dh_boundary;
  a.dOp = w.dOp;
  a.dy = w.dy;
  a.dhc = w.dhc;
  a.slot = w.slot;
  a.rep_dq = w.rep_dq; a.rep_dk = w.rep_dk; a.rep_dg = w.rep_dg; a.rep_dv = w.rep_dv;
  a.rep_db = w.rep_db;
  a.gmax = w.gmax;
  a.n_rounds = p.n_rounds;
  hipError_t e = kda::run_bwd(a, in_dtype == KDA_DTYPE_BF16, p.B, dk, p, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "kda_tree_bwd launch");
  return KDA_OK;
}

int kda_set_overlap(int32_t enable) {
  kda::set_overlap(enable != 0);
  return KDA_OK;
}

namespace {
bool router_shape_ok(int32_t E) { return E == 64 || E == 128 || E == 256 || E == 512; }
}  // namespace

size_t moe_router_workspace_bytes(int64_t n_rows, int32_t n_experts) {
  if (n_rows < 0 || !router_shape_ok(n_experts)) return 0;
  return kda::router_ws_bytes(n_rows, n_experts);
}

int moe_router_stats(const void* logits, int32_t dtype, int64_t n_rows, int32_t n_experts,
                     int32_t top_k, const int32_t* row_mult, int32_t* topk_idx, float* topk_prob,
                     int64_t* load, float* psum, float* zsum, int64_t* n_tok, void* ws,
                     size_t ws_bytes, void* stream) {
  if (dtype != KDA_DTYPE_BF16 && dtype != KDA_DTYPE_FP32) return fail(KDA_ERR_SHAPE, "dtype");
  if (!router_shape_ok(n_experts)) return fail(KDA_ERR_SHAPE, "n_experts must be 64, 128, 256 or 512");
  if (top_k < 1 || top_k > 32 || top_k > n_experts) return fail(KDA_ERR_SHAPE, "top_k");
  if (n_rows < 0 || n_rows >= (int64_t)INT32_MAX) return fail(KDA_ERR_ARG, "bad n_rows");
  if ((n_rows > 0 && (!logits || !row_mult)) || !load || !psum || !zsum || !n_tok || !ws)
    return fail(KDA_ERR_ARG, "null argument");
  if (ws_bytes < kda::router_ws_bytes(n_rows, n_experts))
    return fail(KDA_ERR_WORKSPACE, "router workspace too small");
  hipError_t e = kda::launch_router_stats(logits, dtype == KDA_DTYPE_BF16, n_rows, n_experts, top_k,
                                          row_mult, topk_idx, topk_prob, load, psum, zsum, n_tok,
                                          ws, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "moe_router_stats launch");
  return KDA_OK;
}

int moe_router_stats_noalloc(const void* logits, int32_t dtype, int64_t n_rows,
                             int32_t n_experts, int32_t top_k, const int32_t* row_mult,
                             int32_t* topk_idx, float* topk_prob, int64_t* load, float* psum,
                             float* zsum, int64_t* n_tok, void* stream) {
  if (dtype != KDA_DTYPE_BF16 && dtype != KDA_DTYPE_FP32) return fail(KDA_ERR_SHAPE, "dtype");
  if (!router_shape_ok(n_experts)) return fail(KDA_ERR_SHAPE, "n_experts must be 64, 128, 256 or 512");
  if (top_k < 1 || top_k > 32 || top_k > n_experts) return fail(KDA_ERR_SHAPE, "top_k");
  if (n_rows < 0 || n_rows >= (int64_t)INT32_MAX) return fail(KDA_ERR_ARG, "bad n_rows");
  if ((n_rows > 0 && (!logits || !row_mult)) || !load || !psum || !zsum || !n_tok)
    return fail(KDA_ERR_ARG, "null argument");
  void* ws = nullptr;
  size_t cap = 0;
  hipError_t e = kda::router_scratch(&ws, &cap);
  if (e != hipSuccess) return hip_fail(e, "moe_router_stats_noalloc scratch lookup");
  const size_t need = kda::router_ws_bytes(n_rows, n_experts);
  if (need > cap)
    return fail(KDA_ERR_WORKSPACE, "moe_router_stats_noalloc: " + std::to_string(need) +
                                       " bytes of scratch needed, the built-in scratch holds " +
                                       std::to_string(cap));
  e = kda::launch_router_stats(logits, dtype == KDA_DTYPE_BF16, n_rows, n_experts, top_k, row_mult,
                               topk_idx, topk_prob, load, psum, zsum, n_tok, ws,
                               (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "moe_router_stats_noalloc launch");
  return KDA_OK;
}

int moe_router_stats_bwd(const void* logits, int32_t dtype, int64_t n_rows, int32_t n_experts,
                         const int32_t* row_mult, const float* g_psum, float g_z, float* dlogits,
                         void* stream) {
  if (dtype != KDA_DTYPE_BF16 && dtype != KDA_DTYPE_FP32) return fail(KDA_ERR_SHAPE, "dtype");
  if (!router_shape_ok(n_experts)) return fail(KDA_ERR_SHAPE, "n_experts must be 64, 128, 256 or 512");
  if (n_rows < 0 || n_rows >= (int64_t)INT32_MAX) return fail(KDA_ERR_ARG, "bad n_rows");
  if (n_rows > 0 && (!logits || !row_mult || !g_psum || !dlogits))
    return fail(KDA_ERR_ARG, "null argument");
  hipError_t e = kda::launch_router_bwd(logits, dtype == KDA_DTYPE_BF16, n_rows, n_experts, row_mult,
                                        g_psum, g_z, dlogits, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "moe_router_stats_bwd launch");
  return KDA_OK;
}

int gather_logprobs(const void* logits, int32_t dtype, int64_t n_rows, int32_t vocab,
                    const int32_t* pos_row, const int32_t* pos_target, int64_t n_pos, float* logp,
                    float* lse, void* stream) {
  if (!logits || !lse || (n_pos > 0 && (!pos_row || !pos_target || !logp)))
    return fail(KDA_ERR_ARG, "null argument");
  if (dtype != KDA_DTYPE_BF16 && dtype != KDA_DTYPE_FP32) return fail(KDA_ERR_SHAPE, "dtype");
  if (vocab <= 0 || n_rows < 0 || n_pos < 0 || n_rows >= (int64_t)INT32_MAX)
    return fail(KDA_ERR_ARG, "bad sizes");
  hipError_t e = kda::launch_gather_fwd(logits, dtype == KDA_DTYPE_BF16, n_rows, vocab, pos_row,
                                        pos_target, n_pos, logp, lse, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "gather_logprobs launch");
  return KDA_OK;
}

int gather_logprobs_bwd(const void* logits, int32_t dtype, int64_t n_rows, int32_t vocab,
                        const float* lse, const int32_t* row_pos_ptr, const int32_t* row_pos_idx,
                        const int32_t* pos_target, const float* dlogp, void* dlogits,
                        void* stream) {
  if (!logits || !lse || !row_pos_ptr || !dlogits) return fail(KDA_ERR_ARG, "null argument");
  if (dtype != KDA_DTYPE_BF16 && dtype != KDA_DTYPE_FP32) return fail(KDA_ERR_SHAPE, "dtype");
  if (vocab <= 0 || n_rows < 0 || n_rows >= (int64_t)INT32_MAX) return fail(KDA_ERR_ARG, "bad sizes");
  hipError_t e = kda::launch_gather_bwd(logits, dtype == KDA_DTYPE_BF16, n_rows, vocab, lse,
                                        row_pos_ptr, row_pos_idx, pos_target, dlogp, dlogits,
                                        (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "gather_logprobs_bwd launch");
  return KDA_OK;
}

// ---- tree-ancestor attention ----

namespace {
kda::AttnArgs make_attn_args(const kda::Plan& p, const void* dev, int H, float scale) {
  const int32_t* b = (const int32_t*)dev;
  const kda::DevLayout& d = p.dev;
  kda::AttnArgs a;
  std::memset(&a, 0, sizeof(a));
  a.seg_row = b + d.att_seg_row;
  a.seg_len = b + d.att_seg_len;
  a.anc_ptr = b + d.att_anc_ptr;
  a.anc = b + d.att_anc;
  a.tile_seg = b + d.att_tile_seg;
  a.tile_off = b + d.att_tile_off;
  a.qorder = b + d.att_qorder;
  a.kq_ptr = b + d.att_kq_ptr;
  a.kq = b + d.att_kq;
  a.kw_tile = b + d.att_kw_tile;
  a.kw_q0 = b + d.att_kw_q0;
  a.kw_nq = b + d.att_kw_nq;
  a.kw_slot = b + d.att_kw_slot;
  a.ks_tile = b + d.att_ks_tile;
  a.ks_slot0 = b + d.att_ks_slot0;
  a.ks_n = b + d.att_ks_n;
  a.H = H;
  a.scale = scale;
  return a;
}
bool attn_shape_ok(int32_t H, int32_t d) { return H > 0 && (d == 64 || d == 128); }
// ws = [row deltas [N][H] fp32 | partial dk, dv [n_slots][H][2][64][d] fp32]
size_t attn_ws_carve(const kda::Plan& p, int H, int d, void* base, float** delta, float** part) {
  Carver c(base);
  float* x = c.take((size_t)p.n_rows * H);
  float* y = c.take((size_t)p.att_n_slots * H * 2 * kda::ATT_TILE * d);
  if (delta) *delta = x;
  if (part) *part = y;
  return c.off;
}
}  // namespace

size_t tree_attn_workspace_bytes(const kda_plan* plan, int32_t H, int32_t d) {
  if (!plan || !attn_shape_ok(H, d)) return 0;
  return attn_ws_carve(plan->p, H, d, nullptr, nullptr, nullptr);
}

int tree_attn_fwd(const kda_plan* plan, const void* dev_plan, int32_t H, int32_t d, float scale,
                  const void* q, const void* k, const void* v, float* o, float* lse, void* stream) {
  if (!(scale > 0.f) || !std::isfinite(scale))
    return fail(KDA_ERR_ARG, "attention scale must be a positive finite number");
  int rc = check_dev_plan(plan, dev_plan);
  if (rc) return rc;
  if (!attn_shape_ok(H, d)) return fail(KDA_ERR_SHAPE, "supported: head dim 64 or 128, H > 0");
  if (!q || !k || !v || !o || !lse) return fail(KDA_ERR_ARG, "null tensor argument");
  if (!aligned16({q, k, v, o}) || ((uintptr_t)lse) % 4)
    return fail(KDA_ERR_ARG, "q, k, v, o must be 16-byte aligned, lse 4-byte aligned");
  const kda::Plan& p = plan->p;
  kda::AttnArgs a = make_attn_args(p, dev_plan, H, scale);
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.o = o;
  a.lse = lse;
  hipError_t e = kda::launch_attn_fwd(a, d, (int)p.att_tile_seg.size(), (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "tree_attn_fwd launch");
  return KDA_OK;
}

int tree_attn_bwd(const kda_plan* plan, const void* dev_plan, int32_t H, int32_t d, float scale,
                  const void* q, const void* k, const void* v, const float* o, const float* lse,
                  const void* dO, float* dq, float* dk, float* dv, void* ws, size_t ws_bytes,
                  void* stream) {
  if (!(scale > 0.f) || !std::isfinite(scale))
    return fail(KDA_ERR_ARG, "attention scale must be a positive finite number");
  int rc = check_dev_plan(plan, dev_plan);
  if (rc) return rc;
  if (!attn_shape_ok(H, d)) return fail(KDA_ERR_SHAPE, "supported: head dim 64 or 128, H > 0");
  if (!q || !k || !v || !o || !lse || !dO || !dq || !dk || !dv || !ws)
    return fail(KDA_ERR_ARG, "null tensor argument");
  if (!aligned16({q, k, v, o, dO, dq, dk, dv, ws}) || ((uintptr_t)lse) % 4)
    return fail(KDA_ERR_ARG, "tensors and ws must be 16-byte aligned, lse 4-byte aligned");
  const kda::Plan& p = plan->p;
  if (ws_bytes < attn_ws_carve(p, H, d, nullptr, nullptr, nullptr))
    return fail(KDA_ERR_WORKSPACE, "attention workspace too small");
  kda::AttnArgs a = make_attn_args(p, dev_plan, H, scale);
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.oc = o;
  a.lsec = lse;
  a.dO = (const uint16_t*)dO;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  attn_ws_carve(p, H, d, ws, &a.delta, &a.part);
  hipError_t e = kda::launch_attn_bwd(a, d, p.n_rows, (int)p.att_tile_seg.size(),
                                      (int)p.att_kw_tile.size(), (int)p.att_ks_tile.size(),
                                      (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "tree_attn_bwd launch");
  return KDA_OK;
}

int kda_state_copy(const float* src, const int32_t* src_idx, float* dst, const int32_t* dst_idx,
                   int32_t n, int64_t elems, void* stream) {
  if (n < 0 || elems < 0 || elems % 4) return fail(KDA_ERR_ARG, "n >= 0 and elems a multiple of 4");
  if (n == 0 || elems == 0) return KDA_OK;
  if (!src || !dst) return fail(KDA_ERR_ARG, "null state argument");
  if (!aligned16({src, dst})) return fail(KDA_ERR_ARG, "state arguments must be 16-byte aligned");
  hipError_t e = kda::launch_state_copy(src, src_idx, dst, dst_idx, n, elems, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "kda_state_copy launch");
  return KDA_OK;
}

int kda_state_sum(const float* src, const int32_t* ptr, const int32_t* idx, int32_t n_dst,
                  int64_t elems, int32_t accumulate, float* dst, void* stream) {
  if (n_dst < 0 || elems < 0 || elems % 4) return fail(KDA_ERR_ARG, "n_dst >= 0 and elems a multiple of 4");
  if (n_dst == 0 || elems == 0) return KDA_OK;
  if (!ptr || !dst) return fail(KDA_ERR_ARG, "null argument");
  if (!aligned16({src, dst})) return fail(KDA_ERR_ARG, "state arguments must be 16-byte aligned");
  hipError_t e = kda::launch_state_sum(src, ptr, idx, n_dst, elems, accumulate ? 1 : 0, dst,
                                       (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "kda_state_sum launch");
  return KDA_OK;
}

}  // extern "C"
