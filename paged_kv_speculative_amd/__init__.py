"""Paged-KV speculative verification for AMD MI355X (gfx950).

Python front end of libpkvspec.so (C ABI in include/pkv_spec.h):

    Pool                   page pool + block tables (alloc/append/rollback/release)
    spec_verify_attention  attention of the verification queries over the pages
    spec_verify_attention_static  the same with the library's static scratch (allocates nothing)
    Pool.verify_append     append the new tokens and verify them in one launch
    spec_accept            acceptance rule, accepted length and next token
    spec_accept_tree       the same rule over a draft tree: accepted branch and next token
    PreparedVerify/VerifyAppend/Accept/TreeAccept  the same launches with arguments marshalled once
    tree_ancestor_masks    draft-tree parent list -> ancestor-or-self bitmasks

Torch tensors carry device memory and streams; all arithmetic runs in the
library's HIP kernels.
"""
from .api import (Pool, VerifyBuffers, AcceptBuffers, PreparedVerify, PreparedVerifyAppend, PreparedAccept,
                  spec_verify_attention, spec_verify_attention_static, spec_accept, tree_ancestor_masks, page_bytes,
                  verify_workspace_size, accept_workspace_size, spec_accept_tree,
                  tree_accept_workspace_size, PreparedTreeAccept)
from ._lib import PkvError, OutOfPages

__all__ = ["Pool", "VerifyBuffers", "AcceptBuffers", "PreparedVerify", "PreparedVerifyAppend", "PreparedAccept",
           "spec_verify_attention", "spec_verify_attention_static", "spec_accept", "spec_accept_tree",
           "tree_accept_workspace_size", "PreparedTreeAccept",
           "tree_ancestor_masks", "page_bytes", "verify_workspace_size", "accept_workspace_size",
           "PkvError", "OutOfPages"]
