// spa_kernels.h -- kernel parameter blocks and launchers (internal to libspa).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "spa_plan.h"

namespace spa {

constexpr int MAX_AVG_TERMS = 512;  // averaged (row, head) pairs per KV head

struct AttnParams {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* page_table;
  int64_t pt_stride;
  int64_t num_slots;
  const int32_t* idx;
  void* o;
  float* lse;
  float* logits;
  const ReqDesc* reqs;
  const WorkItem* items;
  float* part_o;
  float* part_ml;
  int32_t Hq, Hkv, G, k;
  float sm_scale;
};

struct MergeParams {
  const ReqDesc* reqs;
  const MergeItem* items;
  const float* part_o;
  const float* part_ml;
  void* o;
  float* lse;
  int32_t Hq, G, k;
};

struct AvgParams {
  const TopkItem* topk;
  const AvgItem* avg;
  const float* logits;
  const float* lse;
  float* pbar;
  int32_t Hq, G, row_begin, row_count;
};

struct SelectParams {
  const TopkItem* topk;
  const float* pbar;
  int32_t* idx;
};

hipError_t launch_attn(const AttnParams& p, int dtype, int head_dim, int nitems, int nthr,
                       size_t smem, hipStream_t st);
hipError_t launch_merge(const MergeParams& p, int dtype, int head_dim, int nitems,
                        hipStream_t st);
hipError_t launch_avg(const AvgParams& ap, int navg, hipStream_t st);
hipError_t launch_select(const SelectParams& sp, int ntopk, hipStream_t st);

}  // namespace spa
