// plan.h -- host-side plan of the tree-packed chunkwise KDA library.
//
// The plan is built once on the host (planner.cpp) from the rollout tree and
// uploaded once as a block of int32 tables; the kernels read only that block.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

namespace kda {

constexpr int32_t ATT_TILE = 64;    // rows per attention query / key tile
constexpr int32_t ATT_KW_MIN = 64;      // query tiles per dk / dv work item, at least
constexpr int32_t ATT_KW_TARGET = 2048; // about this many work items in all

// Offsets (in int32 elements) of each device table inside the uploaded block.
struct DevLayout {
  int64_t round_seq_ptr, seq_chunk_ptr, seq_row_ptr, seq_init_kind, seq_init_idx, seq_leaf, seq_lpt;
  int64_t chunk_seq, chunk_row0, chunk_len, chunk_save, chunk_nrep, chunk_rep0, chunk_round;
  int64_t row_index, out_row;
  int64_t buf_cons_ptr, buf_cons, buf_chunk;
  int64_t rep_row, rep_ptr, rep_slot;
  int64_t root_seq_ptr, root_seq;
  int64_t pos_row, pos_next_row, row_pos_ptr, row_pos_idx, row_mult;
  int64_t att_seg_row, att_seg_len, att_anc_ptr, att_anc, att_seg_tile0;
  int64_t att_tile_seg, att_tile_off, att_qorder, att_kq_ptr, att_kq;
  int64_t att_kw_tile, att_kw_q0, att_kw_nq, att_kw_slot, att_ks_tile, att_ks_slot0, att_ks_n;
  int64_t total;  // int32 elements
};

struct Plan {
  int32_t mode = 0, B = 0, n_seg = 0, n_rounds = 0, n_root = 0, n_leaf = 0;
  int64_t n_rows = 0, n_packed = 0, n_out_rows = 0, R = 0, n_expanded = 0;
  int32_t max_seq_per_round = 0;
  int32_t att_n_slots = 0;  // partial dk / dv slots of split key tiles
  int32_t att_kw_max = 0;   // query tiles per work item, at most

  // per segment
  std::vector<int64_t> seg_start, seg_end;
  std::vector<int32_t> seg_round, seg_seq, seg_is_cont, seg_b, seg_replay;
  // per round
  std::vector<int32_t> round_seq_ptr;
  // per sequence
  std::vector<int32_t> seq_round, seq_head, seq_leaf, seq_b_head, seq_replay;
  std::vector<int32_t> seq_init_kind, seq_init_idx, seq_chunk_ptr;
  std::vector<int32_t> seq_lpt;      // launch order within each round (most chunks first)
  std::vector<int32_t> seq_row_ptr;  // packed rows fit int32 (checked)
  // per chunk
  std::vector<int32_t> chunk_seq, chunk_row0, chunk_len, chunk_save, chunk_nrep, chunk_rep0;
  std::vector<int32_t> chunk_round;   // round of the chunk's sequence
  // per packed row
  std::vector<int32_t> row_index, out_row;
  // handoff buffers
  std::vector<int32_t> buf_seq, buf_chunk, buf_cons_ptr, buf_cons;
  std::vector<int64_t> buf_pos;
  // fixed-order reductions of replay-row gradients into compact rows
  std::vector<int32_t> rep_row, rep_ptr, rep_slot;
  // sequences started from each root's h0 (fixed-order dh0 reduction)
  std::vector<int32_t> root_seq_ptr, root_seq;
  // gather map
  std::vector<int32_t> pos_row, pos_next_row, row_pos_ptr, row_pos_idx;
  // occurrence count of every compact row (trajectories through it)
  std::vector<int32_t> row_mult;
  std::vector<int32_t> leaf_seg, root_seg;
  // tree-ancestor attention.  Tiles are ATT_TILE-row pieces of segments, in
  // canonical order (segment ascending, offset ascending; seg_tile0 is the
  // CSR).  Forward / dq: one block per query tile, in qorder (most keys first).
  // dk / dv: the query tiles that see key tile t are kq[kq_ptr[t] ..] (own
  // segment from t on, then the descendants' tiles in pre-order); they are cut
  // into work items of at most att_kw_max query tiles (kw_*: key tile, first
  // entry, count, partial slot or -1 when the item is the tile's only one);
  // split tiles (ks_*) sum their slots in a fixed order.
  std::vector<int32_t> att_seg_row, att_seg_len, att_anc_ptr, att_anc, att_seg_tile0;
  std::vector<int32_t> att_tile_seg, att_tile_off, att_qorder, att_kq_ptr, att_kq;
  std::vector<int32_t> att_kw_tile, att_kw_q0, att_kw_nq, att_kw_slot, att_ks_tile, att_ks_slot0, att_ks_n;

  DevLayout dev{};
  std::vector<int32_t> dev_blob;  // staged copy of the device block

  int32_t n_seq() const { return (int32_t)seq_round.size(); }
  int32_t n_chunks() const { return (int32_t)chunk_seq.size(); }
  int32_t n_buf() const { return (int32_t)buf_seq.size(); }
};

// Builds a plan; returns 0 or a negative status with `err` set.
int build_plan(int32_t n_seg, const int32_t* parent, const int32_t* seg_len,
               const int64_t* seg_row, int32_t chunk, int32_t mode, Plan& out, std::string& err);

}  // namespace kda
