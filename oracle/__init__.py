"""fp64 CPU oracle for local cluster attention over off-grid tokens.

TEST INFRASTRUCTURE ONLY.  This package is imported by ``tests/``, by
``__graft_entry__.smoke()`` and by the ``cpu_baseline`` leg of ``bench.py``;
the product path (``gathered_local_attention_amd``) never imports, calls or
links it, and it imports nothing from the product path.

See :mod:`oracle.cluster_attention` (neighbour build and attention) and
:mod:`oracle.knn_sampler` (the decoder's KNN-cache point sampler) and
:mod:`oracle.token_merge` (adaptive off-grid token merging) and
:mod:`oracle.volume` (the neighbour build for 3D tokens) for the
functions and the passages of the pages each one follows.
"""

from .cluster_attention import (  # noqa: F401
    quantize,
    morton_code,
    balanced_clusters,
    centroid_sums,
    cluster_rows,
    centroid_keys,
    nearest_clusters,
    nearest_clusters_fullsort,
    key_lists,
    build_neighbors,
    build_image,
    build_neighbors_varlen,
    count_matrix,
    attn_fwd_dense,
    attn_fwd_gathered,
    attn_bwd_dense,
    attn_bwd_gathered,
)
from .knn_sampler import (  # noqa: F401
    knn_table,
    knn_table_cells,
    query_cells,
    knn_weights,
    knn_sample_fwd,
    knn_sample_bwd,
    knn_table_batch,
    knn_sample_fwd_batch,
    knn_sample_bwd_batch,
)
from .token_merge import (  # noqa: F401
    merge_anchors,
    merge_assign,
    merge_assign_tree,
    merge_weights,
    merge_fwd,
    merge_bwd,
)
from .volume import (  # noqa: F401
    quantize3,
    morton_code3,
    build_image3,
    build_neighbors_3d,
    build_neighbors_varlen_3d,
)
