/*
 * CPU reference ("oracle") for the paged KV-cache varlen attention path.
 * TEST INFRASTRUCTURE ONLY: declared for the ctypes binding in oracle/__init__.py.
 * All arrays are host memory; bf16 values are passed as their uint16 bits.
 */
#ifndef PA_ORACLE_H
#define PA_ORACLE_H
#include <stddef.h>
#include <stdint.h>

size_t oracle_k_index(int64_t n, int64_t g, int64_t t, int64_t d, int64_t Hkv,
                      int64_t bs, int64_t D);
size_t oracle_v_index(int64_t n, int64_t g, int64_t t, int64_t d, int64_t Hkv,
                      int64_t bs, int64_t D);
void oracle_write_kv(uint16_t *k_cache, uint16_t *v_cache, const uint16_t *k,
                     const uint16_t *v, const int64_t *slot_mapping,
                     int64_t num_tokens, int64_t Hkv, int64_t bs, int64_t D);
void oracle_gather_kv(const uint16_t *k_cache, const uint16_t *v_cache,
                      const int32_t *block_tables, int64_t bt_stride,
                      const int32_t *seq_lens, int64_t num_seqs, int64_t Hkv,
                      int64_t bs, int64_t D, uint16_t *k_out, uint16_t *v_out);
void oracle_attend(const uint16_t *q, const uint16_t *k_cache,
                   const uint16_t *v_cache, const int32_t *block_tables,
                   int64_t bt_stride, const int32_t *seq_lens,
                   const int32_t *query_start_loc, int64_t num_seqs,
                   int64_t Hq, int64_t Hkv, int64_t bs, int64_t D, float scale,
                   int64_t max_seq_len, double *scratch, double *out,
                   int nthreads);
void oracle_attend_rows(const uint16_t *q, const uint16_t *k_cache,
                        const uint16_t *v_cache, const int32_t *block_tables,
                        int64_t bt_stride, const int32_t *seq_lens,
                        const int32_t *query_start_loc, int64_t num_seqs,
                        int64_t Hq, int64_t Hkv, int64_t bs, int64_t D,
                        float scale, int64_t max_seq_len, const int64_t *rows,
                        int64_t num_rows, double *scratch, double *out_rows,
                        int nthreads);
void oracle_attend_dense(const uint16_t *q, const uint16_t *k_dense,
                         const uint16_t *v_dense, const int32_t *seq_lens,
                         const int32_t *query_start_loc, int64_t num_seqs,
                         int64_t Hq, int64_t Hkv, int64_t D, float scale,
                         int64_t max_seq_len, double *scratch, double *out);
double oracle_e4m3_decode(uint8_t b);
uint8_t oracle_e4m3_encode(float v);
size_t oracle_k8_index(int64_t n, int64_t g, int64_t t, int64_t d, int64_t Hkv,
                       int64_t bs, int64_t D);
size_t oracle_v8_index(int64_t n, int64_t g, int64_t t, int64_t d, int64_t Hkv,
                       int64_t bs, int64_t D);
void oracle_write_kv_fp8(uint8_t *k_cache, uint8_t *v_cache, const uint16_t *k,
                         const uint16_t *v, const int64_t *slot_mapping,
                         int64_t num_tokens, int64_t Hkv, int64_t bs, int64_t D,
                         float k_scale, float v_scale);
void oracle_attend_fp8(const uint16_t *q, const uint8_t *k8, const uint8_t *v8,
                       float k_scale, float v_scale,
                       const int32_t *block_tables, int64_t bt_stride,
                       const int32_t *seq_lens, const int32_t *query_start_loc,
                       int64_t num_seqs, int64_t Hq, int64_t Hkv, int64_t bs,
                       int64_t D, float scale, int64_t max_seq_len,
                       const int64_t *rows, int64_t num_rows, double *scratch,
                       double *out, int nthreads);
void oracle_copy_blocks(uint8_t *k_cache, uint8_t *v_cache, int64_t block_bytes,
                        int64_t num_blocks, const int64_t *mapping,
                        int64_t num_pairs);
void oracle_expand_block_tables(const int32_t *in, int64_t num_seqs,
                                int64_t in_stride, int64_t bs, int32_t *out);
size_t oracle_mla_index(int64_t n, int64_t t, int64_t d);
void oracle_mla_write_kv(uint16_t *cache, const uint16_t *kv,
                         const int64_t *slot_mapping, int64_t num_tokens);
void oracle_mla_decode(const uint16_t *q, const uint16_t *cache,
                       const int32_t *block_tables, int64_t bt_stride,
                       const int32_t *seq_lens, const int32_t *query_start_loc,
                       int64_t num_seqs, int64_t Hq, float scale, double *out,
                       int nthreads);
int oracle_abi_version(void);
#endif
