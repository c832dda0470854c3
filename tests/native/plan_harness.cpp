// Host-only driver of the library's planning and validation code, built with the address and
// undefined-behaviour sanitizers by tests/test_host_sanitizers.py (the library's host layer
// compiled on its own, no HIP). It reads cases from stdin, one per line:
//
//   P <the 21 kv_attn_params fields in declaration order> <num_cus> <paged 0|1>
//       -> "P <validate_layout status> <make_plan status> <num_splits> <split_tiles>
//           <grid_split> <grid_merge> <variant> <group_padded> <wave_heads> <workspace_bytes>"
//   V <the 21 kv_attn_params fields> <paged 0|1> <batch ctx_lens>
//       [<batch * max_blocks_per_seq table entries>]
//       -> "V <kv_attn_validate_host status>"
//   S <status code>  -> "S <kv_attn_status_string(code)>"
//
// The fields are read into exactly-sized buffers, so any read or write out of bounds inside the
// library code is reported by the sanitizers.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "kv_attn_internal.h"

namespace {

constexpr int kParamFields = 21;

// The 21 fields of kv_attn_params in declaration order; scale is read as a floating-point token
// (so "nan" and "inf" reach the library's check), every other field as an integer.
bool read_params(kv_attn_params* p) {
  char tok[64];
  long long f[kParamFields];
  double scale = 0.0;
  for (int i = 0; i < kParamFields; ++i) {
    if (scanf("%63s", tok) != 1) return false;
    if (i == 10)
      scale = strtod(tok, nullptr);
    else
      f[i] = strtoll(tok, nullptr, 10);
  }
  memset(p, 0, sizeof(*p));
  p->batch = int32_t(f[0]);
  p->num_q_heads = int32_t(f[1]);
  p->num_kv_heads = int32_t(f[2]);
  p->head_dim = int32_t(f[3]);
  p->block_size = int32_t(f[4]);
  p->max_blocks_per_seq = int32_t(f[5]);
  p->max_ctx_len = int32_t(f[6]);
  p->num_splits = int32_t(f[7]);
  p->q_dtype = int32_t(f[8]);
  p->kv_dtype = int32_t(f[9]);
  p->scale = float(scale);
  p->window = int32_t(f[11]);
  p->num_blocks = f[12];
  p->k_stride_block = f[13];
  p->k_stride_token = f[14];
  p->k_stride_head = f[15];
  p->v_stride_block = f[16];
  p->v_stride_token = f[17];
  p->v_stride_head = f[18];
  p->num_sinks = int32_t(f[19]);
  p->num_queries = int32_t(f[20]);
  return true;
}

}  // namespace

int main() {
  char tag[4];
  while (scanf("%3s", tag) == 1) {
    if (tag[0] == 'P') {
      kv_attn_params p;
      int cus = 0, paged = 0;
      if (!read_params(&p) || scanf("%d %d", &cus, &paged) != 2) return 2;
      const kv_attn_status lay = kvattn::validate_layout(&p, paged != 0);
      kvattn::Plan plan;
      memset(&plan, 0, sizeof(plan));
      const kv_attn_status st = kvattn::make_plan(&p, cus, &plan);
      if (st == KV_ATTN_OK)
        printf("P %d %d %d %d %lld %lld %d %d %d %llu\n", int(lay), int(st), plan.num_splits,
               plan.split_tiles, (long long)plan.grid_split, (long long)plan.grid_merge,
               plan.variant, plan.group_padded, plan.wave_heads,
               (unsigned long long)plan.workspace_bytes);
      else
        printf("P %d %d\n", int(lay), int(st));
    } else if (tag[0] == 'V') {
      kv_attn_params p;
      int paged = 0;
      if (!read_params(&p) || scanf("%d", &paged) != 1) return 2;
      const int64_t batch = p.batch > 0 ? p.batch : 0;
      std::vector<int32_t> ctx(static_cast<size_t>(batch));
      for (auto& c : ctx)
        if (scanf("%d", &c) != 1) return 2;
      std::vector<int32_t> table;
      if (paged) {
        const int64_t n = batch * (p.max_blocks_per_seq > 0 ? p.max_blocks_per_seq : 0);
        table.resize(size_t(n));
        for (auto& t : table)
          if (scanf("%d", &t) != 1) return 2;
      }
      const kv_attn_status st =
          kv_attn_validate_host(paged ? table.data() : nullptr, ctx.data(), &p);
      printf("V %d\n", int(st));
    } else if (tag[0] == 'S') {
      int code = 0;
      if (scanf("%d", &code) != 1) return 2;
      printf("S %s\n", kv_attn_status_string(code));
    } else {
      return 2;
    }
  }
  return 0;
}
