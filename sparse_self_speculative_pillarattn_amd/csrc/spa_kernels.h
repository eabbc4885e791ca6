// spa_kernels.h -- kernel parameter blocks and launchers (internal to libspa).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "spa_plan.h"

namespace spa {

struct AttnParams {
  const Item* items;  // pinned host plan, read in place
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* page_table;
  int64_t pt_stride;
  int64_t num_slots;
  const int32_t* idx_in;  // draft lists
  void* o;
  float* lse;
  float* logits;
  void* part_o;        // split-K partial outputs, normalised, in the output type [part_rows][d]
  float* part_ml;
  int32_t Hq, Hkv, G, k;
  float sm_scale;
  uint32_t* ticket;    // item counter of this launch (workspace; zero before, zero after)
  int32_t n_items;     // records at items; set by launch_attn
  int32_t first_static;  // workgroup b starts on item b without a draw; set by launch_attn
  // The post-pass and selection records of the call, copied by this launch
  // from the pinned plan into the workspace (plan_n16 16-byte pieces; 0 = no
  // copy), so that the short launches after it read them from device memory.
  const uint4* plan_src;
  uint4* plan_dst;
  int32_t plan_n16;
  // Workspace the same workgroups clear (zero_n16 16-byte pieces): the
  // selected rows' score histograms that the post-pass then adds to.
  uint4* zero_dst;
  int32_t zero_n16;
  // When set (only when plan_n16 is 0), the workgroup that draws the last
  // ticket stores done_val there (the plan buffer's header, pinned host
  // memory): every workgroup has then read its last plan record, so the host
  // may reuse the plan buffer.
  uint64_t* done;
  uint64_t done_val;
};

struct PostParams {
  const PostItem* items;  // pinned host plan read in place, or its workspace copy
  const void* part_o;  // split-K partial outputs (see AttnParams)
  const float* part_ml;
  void* o;
  float* lse;
  const float* logits;
  float* pbar;
  int32_t Hq, G;
  int32_t avg_row_begin, avg_row_count;
  // Read the logits with plain loads (they are expected in the caches) rather
  // than with the streaming hint.
  bool logits_cached;
  // Selected rows' score histograms (zeroed by the attention launch), added
  // to by the averaging items of rows with hist_slot >= 0; null: none kept.
  uint32_t* hist;
  // When set, the launch stores done_val there (the plan buffer's header) as
  // it starts: the attention launch before it, the last reader of the call's
  // pinned plan, has then finished, so the host may reuse the plan buffer.
  uint64_t* done;
  uint64_t done_val;
  // A call without an attention launch (top-K alone): the post-pass reads its
  // own records from the pinned plan and copies the selection's records
  // (plan_n16 16-byte pieces) into the workspace, where the selection launch
  // reads them; 0 = no copy.
  const uint4* plan_src;
  uint4* plan_dst;
  int32_t plan_n16;
};

struct SelectParams {
  const PostItem* items;  // one POST_AVG record of each selected (r, g)
  const float* pbar;
  int32_t* idx_out;
  const uint32_t* hist;   // [slots][HIST_BINS] counts of the selected rows, or null
  int bm_bits;            // LDS position bitmap of long rows (select_bitmap_bits), 0 for none
  // Chunked long rows (n_chunks records; 0 for none).  The per-row launch's
  // workgroups of chunked rows return at once; the count and chunk launches
  // run one workgroup per chunk record.
  const SelChunk* chunks;
  int32_t n_sel, n_chunks;
  uint32_t* row_info;     // [hist slots][4]: boundary bin << HIST_SHIFT, rank in it, its count
  uint32_t* cand_key;     // [n_chunks][SEL_CAND_CAP] each chunk's boundary-bin keys
  int32_t* cand_pos;      // [n_chunks][SEL_CAND_CAP] and their positions
  uint32_t* cnt_above;    // [n_chunks] keys above the boundary bin in each chunk
  uint32_t* cnt_bin;      // [n_chunks] keys in the boundary bin in each chunk
  // When set, the launch stores done_val there as it starts (the post-pass
  // before it was the call's last reader of the pinned plan).
  uint64_t* done;
  uint64_t done_val;
};

struct RecallParams {
  const RecallReq* reqs;  // pinned host plan, read in place
  const int32_t* idx_in;
  int32_t* idx_out;
  int32_t Hkv;
  int32_t n_sink, n_recent;
};

struct QualityParams {
  const QualityReq* reqs;  // pinned host plan, read in place
  const float* logits;
  const float* lse;
  const int32_t* list;
  float* p;                // workspace: the scored rows' softmax
  int32_t* top;            // [B][H_q][T]
  float* coverage;         // [B][H_q]
  float* recall;           // [B][H_q]
  int32_t Hq, G, row, T;
};

// LDS bytes the attention kernel needs for a launch shape.
size_t attn_smem_bytes(int dtype, int head_dim, int G, int nthr, bool mfma, bool valu,
                       int max_chunk);
size_t post_smem_bytes(int avg_terms, int max_nchunk, bool hist);

hipError_t launch_attn(const AttnParams& p, int dtype, int head_dim, int nitems, int nthr,
                       size_t smem, bool draft, hipStream_t st);
hipError_t launch_post(const PostParams& p, int dtype, int head_dim, int nitems, size_t smem,
                       hipStream_t st);
hipError_t launch_select(const SelectParams& sp, int nitems, hipStream_t st);
hipError_t launch_select_count(const SelectParams& sp, hipStream_t st);
hipError_t launch_select_chunks(const SelectParams& sp, hipStream_t st);
int select_bitmap_bits(int max_len);
// LDS bytes of the recallable-index launch for the longest context of a batch.
size_t recall_smem_bytes(int max_len);
size_t quality_smem_bytes(int max_len);
hipError_t launch_quality(const QualityParams& qp, int nblocks, size_t smem, hipStream_t st);
hipError_t launch_recall(const RecallParams& rp, int nblocks, size_t smem, hipStream_t st);
// One thread stores val at done (the plan buffer's header), after the work
// queued before it on `st`.
hipError_t launch_release(uint64_t* done, uint64_t val, hipStream_t st);

}  // namespace spa
