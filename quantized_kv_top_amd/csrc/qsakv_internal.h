// Host-side launch interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qsakv.h"

namespace qsakv {

enum Kind : int { kInt8 = 0, kInt8Inline = 1, kE4M3 = 2, kBF16 = 3, kNvfp4 = 4 };
enum DType : int { kDtBF16 = 0, kDtFP16 = 1, kDtFP32 = 2 };

// Everything a write kernel needs; validated by the caller.
struct WriteParams {
  const void* k_src;
  const void* v_src;
  const int64_t* slot_mapping;
  uint8_t* k;
  uint8_t* v;
  float* kv_scale;        // INT8: float32 (K, V) per row; NVFP4: block-scale bytes
  float k_scale;          // E4M3 and NVFP4 per-layer scales
  float v_scale;
  int64_t num_tokens;
  int64_t num_slots;      // NB * BS
  int32_t num_kv_heads;
  int32_t src_dtype;
};

hipError_t launch_kv_write(int kind, int head_dim, const WriteParams& p, hipStream_t s);

// Calibration statistics of one tensor; thresholds are float32 bit patterns
// of |x| (the smallest |x| whose quotient by the scale is > 448, >= 2^-9,
// >= 2^-6), derived on the host.
struct CalibParams {
  const void* x;
  int64_t n;
  int32_t src_dtype;
  uint32_t t_sat, t_sub, t_norm;
  void* workspace;
  qkv_calib_result* out;
  int32_t grid1;          // streaming workgroups (set by the launcher)
};

size_t calib_workspace_bytes();
hipError_t launch_calib(const CalibParams& p, hipStream_t s);

// Top-k selection from indexer scores; validated by the caller.
struct TopkParams {
  const void* scores;     // [num_rows][row_stride]
  const int32_t* row_len; // [num_rows]
  int32_t* out;           // [num_rows][topk]
  int32_t num_rows;
  int32_t row_stride;     // elements; a multiple of the scores per 16 bytes
  int32_t topk;
  int32_t seg_len;        // > 0: long rows split into segments of this length
  int32_t row_slots;      // segments * topk rounded up to 4: workspace entries per row
  uint32_t* ws_key;       // segments' lists [num_rows][row_slots] (seg_len > 0)
  int32_t* ws_pos;
};

// Segment length that qsa_topk_select splits rows of this stride into (0: none).
int topk_segment_len(int64_t row_stride, int32_t topk);
hipError_t launch_topk(int src_dtype, const TopkParams& p, hipStream_t s);

// Everything an attention kernel needs; validated by the caller.
struct AttnParams {
  const void* q;
  const int32_t* row_seq;
  const int32_t* block_table;
  const int32_t* topk_idx;
  void* out;
  float* lse;             // may be null
  const uint8_t* k;
  const uint8_t* v;
  const float* kv_scale;  // INT8 side layout; NVFP4 block-scale bytes
  float* ws_o;            // split-K partials [R][Hq][P][D]   (P > 1)
  float* ws_ml;           // split-K (max, sum) [R][Hq][P][2] (P > 1)
  float sm_log2e;         // sm_scale * log2(e)
  float k_scale;          // E4M3 / NVFP4 per-layer scales (1 otherwise)
  float v_scale;
  int32_t q_dtype;
  int32_t out_dtype;
  int32_t num_rows;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;          // Hq / Hkv
  int32_t num_seqs;
  int32_t bt_stride;
  int32_t topk;
  int32_t num_blocks;
  int32_t log2_bs;
  int32_t num_splits;     // P
  int32_t chunk;          // ceil(topk / P)
};

// One pass over every (row, KV head, partition); P == 1 writes out/lse
// directly, P > 1 writes partials that launch_merge combines.
hipError_t launch_attn(int kind, int head_dim, const AttnParams& p, hipStream_t s);
hipError_t launch_merge(int head_dim, const AttnParams& p, hipStream_t s);

}  // namespace qsakv
