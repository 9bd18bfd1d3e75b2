// common.h -- shared device-side declarations of the KDA tree kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

// Device views of the uploaded plan tables (int32).
struct DevPlan {
  const int* round_seq_ptr;
  const int* seq_chunk_ptr;
  const int* seq_row_ptr;
  const int* seq_init_kind;
  const int* seq_init_idx;
  const int* seq_leaf;
  const int* chunk_seq;
  const int* chunk_row0;
  const int* chunk_len;
  const int* chunk_save;
  const int* chunk_nrep;
  const int* chunk_rep0;
  const int* row_index;
  const int* out_row;
  const int* buf_cons_ptr;
  const int* buf_cons;
  const int* buf_chunk;
  const int* rep_row;
  const int* rep_ptr;
  const int* rep_slot;
  const int* root_seq_ptr;
  const int* root_seq;
};

// Chunk-local decay products kept from the forward for the reverse pass, one
// block per (chunk, head), fp16: A [BC][BC], P [BC][BC], and the inverses of
// the 16x16 diagonal blocks of I + diag(beta) A, [BC/16][16][16].
constexpr __host__ __device__ size_t prep_halves(int BC) {
  return (size_t)2 * BC * BC + (size_t)16 * BC;
}

struct FwdArgs {
  DevPlan plan;
  int H;
  float scale;
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* beta;
  const float* h0;     // may be null
  float* o;
  float* h_leaf;
  float* chunk_h;      // [n_chunks,H,D,D]
  float* bufs;         // [n_buf,H,D,D]
  _Float16* prep;      // [n_chunks,H,prep_halves(BC)]
};

struct BwdArgs {
  DevPlan plan;
  int H;
  float scale;
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* beta;
  const float* chunk_h;   // saved start state per chunk [n_chunks,H,D,D]
  const _Float16* prep;   // saved chunk decay products [n_chunks,H,prep_halves(BC)]
  const void* dO;
  const float* dh_leaf;   // may be null
  float* dq;
  float* dk;
  float* dv;
  float* dg;
  float* dbeta;
  float* dh0;
  float* dh_boundary;     // may be null
  float* dy;              // [n_packed,H,D]
  float* dhc;             // [n_chunks,H,D,D] gradient of each chunk's end state
  float* slot;            // [n_seq,H,D,D] gradient of each sequence's start state
  float* rep_dq;          // [n_replay,H,D] gradients of replayed rows
  float* rep_dk;
  float* rep_dg;
  float* rep_dv;
  float* rep_db;          // [n_replay,H]
};

inline __device__ float ld_in(const float* p, size_t i) { return p[i]; }
inline __device__ float ld_in(const uint16_t* p, size_t i) {
  return __uint_as_float(((uint32_t)p[i]) << 16);
}

}  // namespace kda
