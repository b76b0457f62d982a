// The whole verification step in three launches: the tree attention (its split
// combine deferred), the logit pass with the combine's rows as extra workgroups of
// the same launch, then the sampler with its walk (at T = 0 the row merge's launch,
// whose wave that finishes a request's last row walks that request).
// Tree-verification notes (zhangshuibai.github.io), "Tree Verification 详解" part
// D.2: the step is the tree-masked target pass plus the verification of part C over
// every node's row; the attention output is not an input of the verification, so
// the combine can finish beside the logit pass.
#include "internal.hpp"
#include "spec_tree.h"

extern "C" int spec_tree_verify_step(const SpecTreeStepArgs* s, void* stream) {
  using namespace spectree;
  if (!s) return SPEC_ERR_INVALID_ARG;
  const bool greedy = s->temperature == 0.0f;
  const int64_t rows = (int64_t)s->batch * s->n_max;
  if (greedy) {  // the walk runs in the logit pass's last launch: its arguments are checked first
    if (!s->tgt_max || !s->tgt_argmax || !s->tokens || !s->parent || !s->n_nodes || !s->accepted_child ||
        !s->term_token)
      return SPEC_ERR_INVALID_ARG;
    if ((s->path_nodes == nullptr) != (s->out_tokens == nullptr) ||
        (s->path_nodes == nullptr) != (s->accept_len == nullptr))
      return SPEC_ERR_INVALID_ARG;
    if (s->batch < 1 || s->n_max < 1 || s->n_max > 64 || s->vocab < 1) return SPEC_ERR_INVALID_ARG;
    if (!s->softmax_workspace || s->softmax_workspace_bytes < spec_tree_softmax_pair_workspace_size(rows, s->vocab))
      return SPEC_ERR_WORKSPACE;
  }
  AttnCombine comb{};
  int rc = attention_launch(s->q, s->k, s->v, s->dtype, s->block_table, s->page_size, s->kv_capacity, s->n_pages,
                            s->ctx_len, s->n_nodes, s->parent, nullptr, s->batch, s->n_max, s->hq, s->hkv,
                            s->head_dim, s->max_kv_len, s->scale, s->attn_out, s->attn_workspace,
                            s->attn_workspace_bytes, s->status, stream, &comb);
  if (rc != SPEC_OK) return rc;
  if (greedy) {
    const GreedyArgs g{s->parent, s->tokens, s->n_nodes, s->tgt_max, s->tgt_argmax, s->n_max, s->vocab,
                       s->accepted_child, s->term_token, s->path_nodes, s->out_tokens, s->accept_len, s->status};
    uint32_t* counters = (uint32_t*)((char*)s->softmax_workspace + softmax_pair_counters_offset(rows, s->vocab));
    rc = softmax_call(s->tgt_logits, rows, s->vocab, 0.0f, s->tgt_max, s->tgt_sumexp, s->tgt_argmax, nullptr,
                      nullptr, nullptr, s->softmax_workspace, s->softmax_workspace_bytes, s->status, stream, &comb, &g,
                      counters);
    if (rc != SPEC_OK) attention_combine_launch(comb, stream);  // (nothing of that call was launched)
    return rc;
  }
  rc = softmax_pair_call(s->tgt_logits, s->temperature, s->dft_logits, s->draft_temperature, rows, s->vocab,
                         s->parent, s->n_nodes, s->n_max, nullptr, nullptr, nullptr, s->tgt_chunk_max,
                         s->tgt_chunk_sum, nullptr, nullptr, s->dft_chunk_max, s->dft_chunk_sum, s->softmax_workspace,
                         s->softmax_workspace_bytes, s->status, stream, &comb);
  if (rc != SPEC_OK) {  // nothing of that call was launched: finish the attention on its own
    attention_combine_launch(comb, stream);
    return rc;
  }
  return spec_tree_reject_sample(s->tgt_logits, s->temperature, s->tgt_max, s->tgt_argmax, s->tgt_chunk_max,
                                 s->tgt_chunk_sum, s->dft_logits, s->draft_temperature, s->dft_chunk_max,
                                 s->dft_chunk_sum, s->tokens, s->parent, s->n_nodes, s->u_accept, s->u_sample,
                                 s->batch, s->n_max, s->vocab, s->accepted_child, s->term_token, s->path_nodes,
                                 s->out_tokens, s->accept_len, s->sample_workspace, s->sample_workspace_bytes,
                                 s->status, stream);
}

extern "C" size_t spec_tree_step_args_size(void) { return sizeof(SpecTreeStepArgs); }
